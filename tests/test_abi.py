"""Host-side checks of the C ABI (no GPU): the library loads, exports every function the header
declares, and rejects bad arguments before launching anything."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dapf8.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|int|size_t)\s+(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    import decode_attention_paged_fp8_amd as dapf8

    return dapf8.lib()


def test_header_declares_the_three_entry_points():
    names = declared_functions()
    for n in ("kv_append", "kv_tag_verify", "paged_decode_attn", "paged_decode_attn_workspace_size",
              "kv_absmax_update", "kv_scale_from_absmax", "dapf8_last_error", "paged_decode_attn_variant"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for n in declared_functions():
        assert hasattr(L, n), n


def test_nm_shows_c_linkage():
    import subprocess

    import decode_attention_paged_fp8_amd as dapf8

    out = subprocess.run(["nm", "-D", "--defined-only", dapf8.lib_path()], capture_output=True, text=True).stdout
    syms = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for n in declared_functions():
        assert n in syms, n                    # unmangled: extern "C"


def test_argument_checks_without_launch(L):
    vp = ctypes.c_void_p
    # Hq not a multiple of Hkv
    rc = L.paged_decode_attn(None, 0, None, None, 0, None, 1, None, None, None, None, None, 0, 1.0, 1, 6, 4, 128, 128,
                             16, 1, 0, None, 0, None)
    assert rc == -1 and b"Hq" in L.dapf8_last_error()
    # B == 0 is a no-op even with null pointers
    rc = L.paged_decode_attn(None, 0, None, None, 0, None, 1, None, None, None, None, None, 0, 1.0, 0, 8, 2, 128, 128,
                             16, 1, 0, None, 0, None)
    assert rc == 0
    # split not a multiple of 32
    rc = L.paged_decode_attn(None, 0, None, None, 0, None, 1, None, None, None, None, None, 0, 1.0, 1, 8, 2, 128, 128,
                             16, 1, 33, None, 0, None)
    assert rc == -1
    # misaligned pointer
    rc = L.paged_decode_attn(vp(16 + 2), 1, vp(256), vp(512), 0, vp(768), 1, vp(1024), vp(1280), vp(1536), None,
                             vp(2048), 1, 1.0, 1, 8, 2, 128, 128, 16, 1, 0, None, 0, None)
    assert rc == -1 and b"aligned" in L.dapf8_last_error()
    # workspace too small (long sequences need partitions)
    rc = L.paged_decode_attn(vp(256), 1, vp(256), vp(512), 0, vp(768), 4096, vp(1024), vp(1280), vp(1536), None,
                             vp(2048), 1, 1.0, 4, 8, 2, 128, 128, 16, 100, 0, None, 0, None)
    assert rc == -3
    assert L.kv_tag_verify(None, 1, None, None, None, 1, None, 0, 16, None) == 0
    assert L.kv_tag_verify(None, 0, None, None, None, 1, None, 1, 16, None) == -1
    assert L.kv_append(None, None, 0, None, None, 0, None, 1, None, None, 0, None, None, None, 1, 1, 64, 16, 16, 1,
                       None) == 0
    # transcode: n = 0 is a no-op; V pools must come in pairs; Dk a multiple of 64
    assert L.kv_transcode_pages(None, None, None, None, None, None, 0, None, None, 1, 64, 16, 16, 1, 1, None) == 0
    assert L.kv_transcode_pages(vp(256), vp(512), vp(768), None, vp(1024), vp(1280), 1, vp(1536), vp(1792), 1, 64,
                                16, 16, 1, 1, None) == -1
    assert L.kv_transcode_pages(vp(256), None, vp(768), None, vp(1024), vp(1280), 1, vp(1536), None, 1, 96, 16, 16,
                                1, 1, None) == -1
    assert L.kv_transcode_pages(vp(256 + 8), None, vp(768), None, vp(1024), vp(1280), 1, vp(1536), None, 1, 64, 16,
                                16, 1, 1, None) == -1
    # checked attention: only the persistent matrix-core shape; B == 0 is a no-op
    assert L.paged_decode_attn_checked(None, 1, None, vp(256), 0, None, 1, None, None, None, None, None, None, None,
                                       1, 1.0, 0, 32, 8, 128, 128, 16, 1, None, 0, None) == 0
    assert L.paged_decode_attn_checked(None, 1, None, vp(256), 0, None, 1, None, None, None, None, None, None, None,
                                       1, 1.0, 1, 8, 8, 64, 64, 16, 1, None, 0, None) == -2
    assert L.paged_decode_attn_checked(None, 1, None, None, 0, None, 1, None, None, None, None, None, None, None,
                                       1, 1.0, 1, 32, 8, 128, 128, 16, 1, None, 0, None) == -2  # shared-KV
    # page allocator: B == 0 no-op; too many requests; expected tags without live tags
    assert L.kv_pages_alloc(None, None, None, 4, None, None, 0, None, None, 1, None, None) == 0
    assert L.kv_pages_alloc(vp(256), vp(512), None, 4, vp(768), vp(1024), 9000, vp(1280), None, 1, vp(1536),
                            None) == -1
    assert L.kv_pages_alloc(vp(256), vp(512), None, 4, vp(768), vp(1024), 1, vp(1280), vp(1792), 1, vp(1536),
                            None) == -1
    assert L.kv_pages_free(vp(256), vp(512), None, 1, 4, vp(768), None) == -1
    assert L.kv_pages_init(None, None, None, 4, None) == -1
    # K rows are stored in 64-byte dimension chunks: Dk must be a multiple of 64
    assert L.kv_append(None, None, 0, None, None, 0, None, 1, None, None, 1, None, None, None, 1, 1, 96, 16, 16, 1,
                       None) == -1
    # the one-launch check and append: no requests and no tokens is a no-op; tokens need a batch;
    # the check's pointers are required; Dk a multiple of 64; tokens need their inputs; alignment
    va = L.kv_tag_verify_append
    assert va(None, 1, None, None, None, 1, None, None, None, 0, None, None, 0, None, None, 0, None, None, 0, 1, 64, 16,
              16, None) == 0
    assert va(None, 1, None, None, None, 1, None, None, None, 0, None, None, 0, None, None, 3, None, None, 0, 1, 64, 16,
              16, None) == -1
    assert va(None, 1, None, None, None, 1, None, None, None, 0, vp(256), None, 0, None, None, 0, None, None, 2, 1, 64,
              16, 16, None) == -1 and b"required" in L.dapf8_last_error()
    ok = [vp(256), 1, vp(512), vp(768), vp(1024), 1, vp(1280)]
    assert va(*ok, None, None, 0, vp(1536), None, 0, None, None, 0, None, None, 2, 1, 96, 16, 16, None) == -1
    assert va(*ok, None, None, 0, vp(1536), None, 0, None, None, 1, vp(1792), None, 2, 1, 64, 16, 16, None) == -1
    assert va(*ok, vp(2048 + 4), None, 0, vp(1536), None, 0, vp(2304), vp(2560), 1, vp(1792), None, 2, 1, 64, 16, 16,
              None) == -1 and b"aligned" in L.dapf8_last_error()


def test_plan_and_workspace(L):
    import decode_attention_paged_fp8_amd as dapf8

    # GQA decode batch: stream-K over all windows, one partition per sequence unless asked
    name, split = dapf8.paged_decode_attn_variant(32, 32, 8, 128, 128, 16, 513)
    assert name == "mfma_streamk_g16_d128_p16" and split == -(-513 * 16 // 32) * 32
    n = dapf8.paged_decode_attn_workspace_size(32, 32, 8, 128, 128, 16, 513)
    assert n >= (32 * 8 + 4096) * 4 * (128 + 4) * 4
    # batches above the stream-K limit use fixed partitions
    name, split = dapf8.paged_decode_attn_variant(2000, 32, 8, 128, 128, 16, 513)
    assert name == "mfma_g16_d128_p16" and split % 256 == 0 and 256 <= split <= 4096
    assert dapf8.paged_decode_attn_variant(4, 8, 8, 64, 64, 16, 13)[0] == "valu_generic"
    # shared-KV latent shape: matrix-core stream-K over 64-token pages; partitions are whole pages
    name, split = dapf8.paged_decode_attn_variant(64, 128, 1, 576, 512, 64, 512, shared_kv=True)
    assert name == "mfma_latent_d576_p64" and split == 512 * 64
    # persistent kernels split work into their own slices: split_tokens does not change the plan
    assert dapf8.paged_decode_attn_variant(64, 128, 1, 576, 512, 64, 512, 96, shared_kv=True)[1] == 512 * 64
    n = dapf8.paged_decode_attn_workspace_size(64, 128, 1, 576, 512, 64, 512, shared_kv=True)
    assert n >= (64 + 512) * 128 * (512 + 4) * 4          # pieces: B*Hkv*nsplit + 512 workgroups
    # a split the generic (fp32-query) fallback cannot take does not fail the bf16-query plan
    assert dapf8.paged_decode_attn_variant(64, 128, 1, 576, 512, 64, 512, 8192, shared_kv=True)[0] == \
        "mfma_latent_d576_p64"
    assert dapf8.paged_decode_attn_workspace_size(64, 128, 1, 576, 512, 64, 512, 8192, shared_kv=True) >= n
    # BF16 storage, unsupported group sizes and other dims stay on the generic kernel
    assert dapf8.paged_decode_attn_variant(64, 128, 1, 576, 512, 64, 512, kv_dt=1, shared_kv=True)[0] == "valu_generic"
    assert dapf8.paged_decode_attn_variant(4, 24, 1, 576, 512, 64, 512, shared_kv=True)[0] == "valu_generic"
    assert dapf8.paged_decode_attn_variant(4, 128, 1, 576, 512, 16, 512, shared_kv=True)[0] == "valu_generic"
    # the long-context case asks for 4096-token partitions: stream-K still uses its own slices,
    # while the fixed-partition and generic kernels honour the request
    name, split = dapf8.paged_decode_attn_variant(8, 64, 8, 128, 128, 16, 16384, 4096)
    assert name == "mfma_streamk_g16_d128_p16" and split == 16384 * 16
    assert dapf8.paged_decode_attn_variant(2000, 32, 8, 128, 128, 16, 513, 4096)[1] == 4096
    assert dapf8.paged_decode_attn_variant(4, 8, 8, 64, 64, 16, 513, 1024)[1] == 1024
    # short sequences on the generic path: one partition, no workspace
    assert dapf8.paged_decode_attn_workspace_size(4, 8, 8, 64, 64, 16, 2) == 0
