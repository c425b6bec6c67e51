// The host side of the C ABI (pa_api.hip: argument checks, launch plans,
// workspace sizes) built with AddressSanitizer and UndefinedBehaviorSanitizer
// on the host.  Every call here is one the library must refuse, or answer,
// before any launch -- null or misaligned pointers, sizes and shapes out of
// range, workspaces too small, workspace and path queries for explicit
// partitions -- so the driver runs the same with or without a GPU and never
// hands a kernel the fake addresses it passes.  Exit status 0 = clean.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "pa.h"
#include "pa_blocks.h"
#include "pa_probe.h"

namespace {

int failures = 0;

void expect(const char *what, int line, int got, int want)
{
    if (got != want) {
        std::fprintf(stderr, "api_driver: %s (line %d): status %d, expected %d\n", what, line, got, want);
        ++failures;
    }
}
#define EXPECT(call, want) expect(#call, __LINE__, (int)(call), (int)(want))

void *const F = reinterpret_cast<void *>(uintptr_t(0x7f0000000000));   // 16-byte aligned, never dereferenced
void *at(uintptr_t off) { return reinterpret_cast<void *>(uintptr_t(0x7f0000000000) + off); }
const int32_t *I(void *p) { return static_cast<const int32_t *>(p); }

struct Dec {
    void *out = F, *q = F, *k = F, *v = F, *bt = F, *cl = F;
    int S = 2, Hq = 4, Hkv = 2, D = 64, bs = 16, MB = 8, NB = 32;
    float scale = 0.125f;
    pa_dtype dt = PA_F16;
    pa_layout layout = PA_LAYOUT_BHTD;
    int pt = PA_PARTITION_SINGLE;
    pa_kernel kern = PA_KERNEL_AUTO;
    unsigned flags = 0;
    void *ws = nullptr;
    size_t wsb = 0;
    pa_status run() const {
        return pa_decode_ex(out, q, k, v, I(bt), I(cl), S, Hq, Hkv, D, bs, MB, NB, scale, dt, layout, pt, kern, flags,
                            ws, wsb, nullptr);
    }
};

}  // namespace

int main()
{
    // decode: every refusal happens before a launch
    {
        Dec d; d.S = 0; d.out = d.q = d.k = d.v = d.bt = d.cl = nullptr; EXPECT(d.run(), PA_OK);
    }
    { Dec d; d.out = nullptr; EXPECT(d.run(), PA_ERR_INVALID_ARG); }
    { Dec d; d.q = nullptr; EXPECT(d.run(), PA_ERR_INVALID_ARG); }
    { Dec d; d.bt = nullptr; EXPECT(d.run(), PA_ERR_INVALID_ARG); }
    { Dec d; d.q = at(8); EXPECT(d.run(), PA_ERR_INVALID_ARG); }
    { Dec d; d.k = at(4); EXPECT(d.run(), PA_ERR_INVALID_ARG); }
    { Dec d; d.cl = at(2); EXPECT(d.run(), PA_ERR_INVALID_ARG); }
    { Dec d; d.scale = NAN; EXPECT(d.run(), PA_ERR_INVALID_ARG); }
    { Dec d; d.scale = INFINITY; EXPECT(d.run(), PA_ERR_INVALID_ARG); }
    { Dec d; d.NB = 0; EXPECT(d.run(), PA_ERR_INVALID_ARG); }
    { Dec d; d.S = -1; EXPECT(d.run(), PA_ERR_INVALID_ARG); }
    { Dec d; d.MB = 0; EXPECT(d.run(), PA_ERR_INVALID_ARG); }
    { Dec d; d.Hq = 5; EXPECT(d.run(), PA_ERR_INVALID_ARG); }
    { Dec d; d.Hkv = 0; EXPECT(d.run(), PA_ERR_INVALID_ARG); }
    { Dec d; d.D = 96; EXPECT(d.run(), PA_ERR_UNSUPPORTED); }
    { Dec d; d.bs = 4; EXPECT(d.run(), PA_ERR_UNSUPPORTED); }
    { Dec d; d.layout = (pa_layout)2; EXPECT(d.run(), PA_ERR_UNSUPPORTED); }
    { Dec d; d.dt = (pa_dtype)9; EXPECT(d.run(), PA_ERR_UNSUPPORTED); }
    { Dec d; d.kern = (pa_kernel)3; EXPECT(d.run(), PA_ERR_UNSUPPORTED); }
    { Dec d; d.kern = PA_KERNEL_MFMA; EXPECT(d.run(), PA_ERR_UNSUPPORTED); }                  // head_dim 64
    { Dec d; d.kern = PA_KERNEL_MFMA; d.D = 128; d.dt = PA_F32; EXPECT(d.run(), PA_ERR_UNSUPPORTED); }
    { Dec d; d.flags = 2; EXPECT(d.run(), PA_ERR_INVALID_ARG); }
    { Dec d; d.pt = 24; EXPECT(d.run(), PA_ERR_INVALID_ARG); }                               // not a block multiple
    { Dec d; d.pt = -3; EXPECT(d.run(), PA_ERR_INVALID_ARG); }
    { Dec d; d.pt = 64; d.MB = 64; EXPECT(d.run(), PA_ERR_WORKSPACE); }
    { Dec d; d.pt = 64; d.MB = 64; d.ws = F; d.wsb = 16; EXPECT(d.run(), PA_ERR_WORKSPACE); }
    { Dec d; d.pt = 64; d.MB = 64; d.ws = at(8); d.wsb = size_t(1) << 30; EXPECT(d.run(), PA_ERR_WORKSPACE); }
    { Dec d; d.MB = (1 << 30) / 16 + 1; EXPECT(d.run(), PA_ERR_UNSUPPORTED); }
    EXPECT(pa_decode(nullptr, F, F, F, I(F), I(F), 2, 4, 2, 64, 16, 8, 0.125f, PA_F16, nullptr, 0, nullptr),
           PA_ERR_INVALID_ARG);
    EXPECT(pa_decode_noalloc(F, F, F, F, I(F), I(F), 2, 4, 2, 96, 16, 8, 0.125f, PA_F16, nullptr), PA_ERR_UNSUPPORTED);
    EXPECT(pa_decode_noalloc(F, at(8), F, F, I(F), I(F), 2, 4, 2, 64, 16, 8, 0.125f, PA_F16, nullptr),
           PA_ERR_INVALID_ARG);
    // decode + append
    EXPECT(pa_decode_append(F, F, nullptr, F, F, F, static_cast<const int64_t *>(F), I(F), I(F), 2, 4, 2, 64, 16, 8,
                            32, 0.125f, PA_F16, PA_LAYOUT_BHTD, -1, PA_KERNEL_AUTO, 0, nullptr, 0, nullptr),
           PA_ERR_INVALID_ARG);
    EXPECT(pa_decode_append(F, F, F, F, F, F, static_cast<const int64_t *>(at(4)), I(F), I(F), 2, 4, 2, 64, 16, 8, 32,
                            0.125f, PA_F16, PA_LAYOUT_BHTD, -1, PA_KERNEL_AUTO, 0, nullptr, 0, nullptr),
           PA_ERR_INVALID_ARG);
    // append
    const int64_t *SM = static_cast<const int64_t *>(F);
    EXPECT(pa_reshape_and_cache(nullptr, nullptr, nullptr, nullptr, nullptr, 0, 2, 64, 16, 8, PA_F16, PA_LAYOUT_BHTD,
                                nullptr), PA_OK);
    EXPECT(pa_reshape_and_cache(nullptr, F, F, F, SM, 3, 2, 64, 16, 8, PA_F16, PA_LAYOUT_BHTD, nullptr),
           PA_ERR_INVALID_ARG);
    EXPECT(pa_reshape_and_cache(F, F, F, F, SM, -1, 2, 64, 16, 8, PA_F16, PA_LAYOUT_BHTD, nullptr), PA_ERR_INVALID_ARG);
    EXPECT(pa_reshape_and_cache(F, F, F, F, SM, 3, 2, 40, 16, 8, PA_F16, PA_LAYOUT_BHTD, nullptr), PA_ERR_UNSUPPORTED);
    EXPECT(pa_reshape_and_cache(F, F, F, F, SM, 3, 2, 64, 16, 0, PA_F16, PA_LAYOUT_BHTD, nullptr), PA_ERR_INVALID_ARG);
    // prefill
    EXPECT(pa_prefill(F, F, F, F, I(F), I(F), I(F), 2, 10, 5, 8, 2, 64, 16, 8, 32, 0.1f, PA_F16, PA_LAYOUT_BHTD, 0,
                      nullptr), PA_ERR_UNSUPPORTED);                                       // head_dim 64
    EXPECT(pa_prefill(F, F, F, F, I(F), I(F), nullptr, 2, 10, 5, 8, 2, 128, 16, 8, 32, 0.1f, PA_F16, PA_LAYOUT_BHTD, 0,
                      nullptr), PA_ERR_INVALID_ARG);
    EXPECT(pa_prefill(F, F, F, F, I(F), I(F), I(F), 2, -1, 5, 8, 2, 128, 16, 8, 32, 0.1f, PA_F16, PA_LAYOUT_BHTD, 0,
                      nullptr), PA_ERR_INVALID_ARG);
    EXPECT(pa_prefill(F, F, F, F, I(F), I(F), I(F), 2, 10, 5, 8, 2, 128, 16, 8, 32, 0.1f, PA_F16, PA_LAYOUT_BHTD, 4,
                      nullptr), PA_ERR_INVALID_ARG);
    // shared-prefix decode
    EXPECT(pa_decode_shared_prefix(F, F, F, F, I(F), I(F), 4, 8, 2, 128, 16, 8, 32, 9, 0.1f, PA_F16, PA_LAYOUT_BHTD,
                                   F, 1 << 20, nullptr), PA_ERR_INVALID_ARG);              // prefix past the table
    EXPECT(pa_decode_shared_prefix(F, F, F, F, I(F), I(F), 4, 8, 2, 128, 16, 8, 32, 4, 0.1f, PA_F16, PA_LAYOUT_BHTD,
                                   F, 16, nullptr), PA_ERR_WORKSPACE);
    EXPECT(pa_decode_shared_prefix(F, F, F, F, I(F), I(F), 4, 8, 2, 128, 16, 8, 32, 4, 0.1f, PA_F32, PA_LAYOUT_BHTD,
                                   F, 1 << 20, nullptr), PA_ERR_UNSUPPORTED);
    // workspace and path queries for explicit partitions (no device needed)
    size_t bytes = 1;
    EXPECT(pa_decode_workspace_bytes(2, 4, 2, 64, 16, 8, PA_F16, PA_PARTITION_SINGLE, &bytes), PA_OK);
    if (bytes != 0)
        ++failures, std::fprintf(stderr, "api_driver: single pass needs no workspace, got %zu\n", bytes);
    EXPECT(pa_decode_workspace_bytes(2, 4, 2, 64, 16, 64, PA_F16, 64, &bytes), PA_OK);
    // 2 seqs x 4 heads x 16 partitions: 128 (max, sum) pairs (1 KiB, a multiple of 256 bytes), then 64 floats each
    if (bytes != (size_t)2 * 4 * 16 * 8 + (size_t)2 * 4 * 16 * 64 * 4)
        ++failures, std::fprintf(stderr, "api_driver: split-K workspace %zu\n", bytes);
    EXPECT(pa_decode_workspace_bytes(2, 4, 2, 64, 16, 64, PA_F16, 64, nullptr), PA_ERR_INVALID_ARG);
    EXPECT(pa_decode_workspace_bytes(2, 4, 2, 64, 16, 64, PA_F16, 40, &bytes), PA_ERR_INVALID_ARG);
    int part = 0;
    pa_kernel kern = PA_KERNEL_AUTO;
    EXPECT(pa_decode_path(2, 64, 8, 128, 16, 64, PA_BF16, 256, PA_KERNEL_AUTO, &part, &kern), PA_OK);
    if (part != 256 || kern != PA_KERNEL_MFMA)
        ++failures, std::fprintf(stderr, "api_driver: path %d/%d\n", part, (int)kern);
    EXPECT(pa_decode_path(2, 4, 4, 64, 16, 64, PA_F16, PA_PARTITION_SINGLE, PA_KERNEL_AUTO, &part, &kern), PA_OK);
    if (part != PA_PARTITION_SINGLE || kern != PA_KERNEL_VECTOR)
        ++failures, std::fprintf(stderr, "api_driver: path %d/%d\n", part, (int)kern);
    EXPECT(pa_decode_path(2, 4, 4, 64, 16, 64, PA_F16, -1, PA_KERNEL_AUTO, nullptr, &kern), PA_ERR_INVALID_ARG);
    // block copies, probe
    EXPECT(pa_copy_blocks(F, F, I(F), 3, 0, 16, 2, 64, PA_F16, nullptr), PA_ERR_INVALID_ARG);
    EXPECT(pa_copy_blocks(F, F, I(at(2)), 3, 8, 16, 2, 64, PA_F16, nullptr), PA_ERR_INVALID_ARG);
    EXPECT(pa_copy_blocks(F, F, I(F), 3, 8, 16, 2, 48, PA_F16, nullptr), PA_ERR_UNSUPPORTED);
    EXPECT(pa_copy_blocks(F, F, I(F), 0, 8, 16, 2, 64, PA_F16, nullptr), PA_OK);
    EXPECT(pa_probe_stream_read(F, 100, static_cast<uint32_t *>(F), 4, 0, nullptr), PA_ERR_INVALID_ARG);
    EXPECT(pa_probe_stream_read(F, 1 << 20, static_cast<uint32_t *>(F), 0, 0, nullptr), PA_ERR_INVALID_ARG);
    EXPECT(pa_probe_stream_read(F, 1 << 20, static_cast<uint32_t *>(F), 4, 3, nullptr), PA_ERR_INVALID_ARG);
    EXPECT(pa_probe_stream_read(F, 3 * 4096, static_cast<uint32_t *>(F), 4, 2, nullptr), PA_ERR_INVALID_ARG);
    // status strings and version
    for (int s = -1; s <= 6; ++s)
        if (!pa_status_string((pa_status)s) || !pa_status_string((pa_status)s)[0])
            ++failures, std::fprintf(stderr, "api_driver: empty status string %d\n", s);
    if (pa_abi_version() < 202)
        ++failures, std::fprintf(stderr, "api_driver: version %d\n", pa_abi_version());
    if (failures) {
        std::fprintf(stderr, "api_driver: %d failures\n", failures);
        return 1;
    }
    std::printf("api_driver: clean\n");
    return 0;
}
