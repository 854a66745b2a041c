// stream_read.hip -- measurement helper: a plain read of a device buffer with
// 16-byte loads under the weight streams' cache policy (kStreamPolicy), the
// ceiling the projection kernels are compared with.  It
// does nothing of the method: every lane loads its 16-byte chunks, folds
// them into one word and stores nothing unless that word has one particular
// value (so the loads cannot be dropped and almost no store is made).
#include "device.h"
#include "tt_internal.h"

namespace tt {

constexpr int kReadThreads = 256;

// Workgroup b reads bytes [b * span, (b + 1) * span) of the buffer, span =
// 256 lanes x 16 bytes x U loads, all U loads of a lane issued before any is
// used.  Loads past the end return zero (buffer descriptor range).
template <int U>
__global__ __launch_bounds__(kReadThreads) void k_stream_read(const uint8_t *buf, int64_t bytes,
                                                              uint32_t *sink) {
    constexpr int64_t span = (int64_t)kReadThreads * 16 * U;
    const int64_t base = (int64_t)blockIdx.x * span;
    const int64_t left = bytes - base;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(buf + base), 0, (int)(left < span ? left : span), 0x00020000);
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
        v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, (u * kReadThreads + threadIdx.x) * 16, 0,
                                                     kStreamPolicy);
    uint32_t x = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    if (x == 0x9E3779B9u) sink[0] = x;
}

}  // namespace tt

using namespace tt;

extern "C" tt_status tt_stream_read(const void *buf, int64_t bytes, int32_t loads_per_lane,
                                    uint32_t *sink, void *stream) {
    TT_TRY(check_ptr(buf, "buf"));
    TT_TRY(check_ptr(sink, "sink"));
    TT_TRY(check_align(buf, 16, "buf"));
    TT_TRY(check_align(sink, 4, "sink"));
    TT_TRY(check_range(bytes, 16, (int64_t)1 << 40, "bytes"));
    if (bytes % 16) return fail(TT_E_SHAPE, "bytes = %lld is not a multiple of 16", (long long)bytes);
    const int U = loads_per_lane;
    if (U != 1 && U != 2 && U != 4 && U != 8)
        return fail(TT_E_SHAPE, "loads_per_lane = %d; 1, 2, 4 or 8", U);
    const int64_t span = (int64_t)kReadThreads * 16 * U;
    const int64_t blocks = ceil_div(bytes, span);
    if (blocks > INT32_MAX) return fail(TT_E_SHAPE, "bytes = %lld is too large", (long long)bytes);
    const uint8_t *b = static_cast<const uint8_t *>(buf);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 grid((unsigned)blocks), block(kReadThreads);
    tt_status st;
    switch (U) {
        case 1: st = launch("stream read", k_stream_read<1>, grid, block, 0, s, b, bytes, sink); break;
        case 2: st = launch("stream read", k_stream_read<2>, grid, block, 0, s, b, bytes, sink); break;
        case 4: st = launch("stream read", k_stream_read<4>, grid, block, 0, s, b, bytes, sink); break;
        default: st = launch("stream read", k_stream_read<8>, grid, block, 0, s, b, bytes, sink); break;
    }
    if (st == TT_OK) clear_error();
    return st;
}
