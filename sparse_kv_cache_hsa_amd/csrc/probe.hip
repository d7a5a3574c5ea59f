// probe.hip -- a measurement helper beside the method: the device's read
// rate for a plain stream of 4 KB chunks and for 4 KB chunks gathered at
// scattered offsets (the access pattern of the decode kernel's K/V stream,
// one page slice of 16 bf16 rows of 128 channels).  The decode kernel's
// bytes per second are read against these rates as well as against the
// HBM specification.
//
// A block of 256 threads reads one 4 KB chunk per pass (one 16-byte
// non-temporal load per thread) and keeps kInFlight chunks in flight; the
// loaded words are folded into an XOR per thread and each wave stores its
// XOR, so no load can be dropped and the stored words XOR to the XOR of
// every word read (which the tests check).
#include "rkv_internal.h"

namespace rkv {
namespace {

constexpr int kProbeBlock = 256;
constexpr int kProbeChunk = kProbeBlock * 16;  // bytes per chunk pass
constexpr int kInFlight = 8;

typedef unsigned int probe_u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(kProbeBlock)
read_probe_kernel(const unsigned char *buf, const int64_t *offsets, int64_t n_chunks,
                  uint32_t *sink) {
    const int tid = threadIdx.x;
    uint32_t acc = 0u;
    const int64_t stride = (int64_t)gridDim.x;
    for (int64_t c0 = blockIdx.x; c0 < n_chunks; c0 += stride * kInFlight) {
        int64_t off[kInFlight];
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) {
            const int64_t c = c0 + u * stride;
            off[u] = c < n_chunks ? (offsets ? offsets[c] : c * kProbeChunk) : -1;
        }
        probe_u32x4 v[kInFlight];
#pragma unroll
        for (int u = 0; u < kInFlight; ++u)
            v[u] = off[u] >= 0 ? __builtin_nontemporal_load(
                                     (const probe_u32x4 *)(buf + off[u] + (int64_t)tid * 16))
                               : probe_u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    acc ^= lane_xor<1>(acc);
    acc ^= lane_xor<2>(acc);
    acc ^= lane_xor<4>(acc);
    acc ^= lane_xor<8>(acc);
    acc ^= lane_xor<16>(acc);
    acc ^= lane_xor<32>(acc);
    if ((tid & (kWave - 1)) == 0) sink[blockIdx.x * (kProbeBlock / kWave) + tid / kWave] = acc;
}

}  // namespace
}  // namespace rkv

using namespace rkv;

extern "C" int rkv_read_probe(const void *buf, const int64_t *offsets, int64_t n_chunks,
                              uint32_t *sink, void *stream) {
    if (!buf || !sink || n_chunks < 1 || ((uintptr_t)buf & 15u) != 0) return RKV_EINVAL;
    static_assert(kProbeChunk == RKV_READ_PROBE_CHUNK, "chunk size");
    clear_pending_error();
    const int blocks = (int)(n_chunks < RKV_READ_PROBE_BLOCKS ? n_chunks : RKV_READ_PROBE_BLOCKS);
    read_probe_kernel<<<blocks, kProbeBlock, 0, (hipStream_t)stream>>>(
        (const unsigned char *)buf, offsets, n_chunks, sink);
    return launch_status();
}
