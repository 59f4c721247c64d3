"""Host-side parsing of rocprofv3 output (no GPU)."""
import pytest

from video_diffusion_transformer_block_amd import profiling


def test_short_name_strips_signature_and_namespaces():
    assert profiling.short_name("void vdtq::hq_nvfp4_kernel<64, false>(vdtq::HQParams)") == "hq_nvfp4_kernel<64, false>"
    assert profiling.short_name(
        "(anonymous namespace)::stream_rows_kernel(HIP_vector_type<unsigned int, 4u> const*, long)") == "stream_rows_kernel"


def test_short_name_tensile_kernel():
    n = "Cijk_Ailk_Bljk_BBS_BH_Bias_HA_S_SAV_UserArgs_MT256x256x64_MI16x16x1_SN_LDSB1"
    assert profiling.short_name(n) == "hipBLASLt Ailk MT256x256x64"


@pytest.mark.parametrize("name", ["__amd_rocclr_fillBufferAligned", "qgemm_reduce_kernel<2>"])
def test_short_name_plain(name):
    assert profiling.short_name(name) == name
