// Reference read kernels for measurement (libpkvprobe.so, loaded by the
// benchmark's --read-ceiling mode only; no decode call uses them).
//
// They give the rate at which this memory delivers a decode's bytes when
// nothing is computed: (1) one contiguous stream of the same number of bytes,
// (2) the decode's own tile pattern: for every (sequence, partition) item and
// KV head, the (block, KV head) tiles of both caches named by the block table,
// one work-group of 4 waves per item and head, each wave a quarter of the
// item's blocks with two tiles in flight, every load 16 bytes per lane and
// nontemporal, and at most 16 waves per compute unit (each work-group holds a
// quarter of the 160 KiB LDS, unused), as in the decode kernels.  Each lane
// folds what it read into a 32-bit XOR and writes it to `sink`, so that no
// load can be dropped; the XOR of the whole sink is the XOR of every 32-bit
// word read (a word read twice cancels), which the tests check.
//
// C ABI (device pointers; returns 0 or the HIP error of the launch, -1 for
// arguments outside what the kernels take):
//   pkvprobe_stream_read(buf, bytes, sink, grid, stream)
//     bytes a multiple of 16; grid work-groups of 256 lanes, work-group b
//     reading the b-th of grid nearly equal contiguous pieces, 8 loads per lane
//     in flight; sink holds grid * 256 words.
//   pkvprobe_tile_read(k_cache, v_cache, block_tables, item_seq, item_first,
//                      item_end, n_items, num_kv_heads, max_blocks_per_seq,
//                      num_blocks, tile_bytes, sink, stream)
//     caches [num_blocks][num_kv_heads][tile_bytes]; item i reads blocks
//     block_tables[item_seq[i]][item_first[i] .. item_end[i] - 1] (entries
//     outside [0, num_blocks) read block 0); tile_bytes 1024, 2048, 4096 or
//     8192; sink holds n_items * num_kv_heads * 256 words.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef unsigned int probe_u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ probe_u32x4 load16(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const probe_u32x4*>(p));
}

__device__ __forceinline__ uint32_t fold(probe_u32x4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

constexpr int kInFlight = 8;                  // loads per lane in flight in the stream

__global__ void __launch_bounds__(256) stream_read_kernel(const uint8_t* p, size_t n16,
                                                          uint32_t* sink) {
  const size_t nb = gridDim.x;
  const size_t per = (n16 + nb - 1) / nb;
  const size_t lo = per * blockIdx.x;
  const size_t hi = lo + per < n16 ? lo + per : n16;
  uint32_t acc = 0;
  size_t i = lo + threadIdx.x;
  for (; i + (kInFlight - 1) * 256 < hi; i += kInFlight * 256) {
    probe_u32x4 t[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) t[u] = load16(p + 16 * (i + u * 256));
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) acc ^= fold(t[u]);
  }
  for (; i < hi; i += 256) acc ^= fold(load16(p + 16 * i));
  sink[size_t(blockIdx.x) * 256 + threadIdx.x] = acc;
}

template <int NLD>                            // 1 KiB loads per tile and cache
__global__ void __launch_bounds__(256) tile_read_kernel(const uint8_t* kc, const uint8_t* vc,
                                                        const int* bt, const int* it_s,
                                                        const int* it_j0, const int* it_j1,
                                                        int Hk, int MB, int NB, uint32_t* sink) {
  constexpr size_t kTile = size_t(NLD) * 1024;
  const int item = blockIdx.x / Hk, h = blockIdx.x % Hk;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int s = it_s[item], pj0 = it_j0[item], pj1 = it_j1[item];
  const int j0 = pj0 + (w * (pj1 - pj0)) / 4, j1 = pj0 + ((w + 1) * (pj1 - pj0)) / 4;
  auto base = [&](const uint8_t* c, int j) {
    int id = bt[size_t(s) * MB + j];
    if (static_cast<unsigned>(id) >= static_cast<unsigned>(NB)) id = 0;
    return c + (size_t(id) * Hk + h) * kTile + lane * 16;
  };
  probe_u32x4 a[2 * NLD], b[2 * NLD];
  uint32_t acc = 0;
  auto load = [&](int j, probe_u32x4 (&t)[2 * NLD]) {
    const uint8_t* kp = base(kc, j);
    const uint8_t* vp = base(vc, j);
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      t[i] = load16(kp + 1024 * i);
      t[NLD + i] = load16(vp + 1024 * i);
    }
  };
  auto use = [&](const probe_u32x4 (&t)[2 * NLD]) {
#pragma unroll
    for (int i = 0; i < 2 * NLD; ++i) acc ^= fold(t[i]);
  };
  int j = j0;
  if (j < j1) load(j, a);
  for (; j + 1 < j1; j += 2) {                // tiles j and j + 1 in flight
    load(j + 1, b);
    use(a);
    if (j + 2 < j1) load(j + 2, a);
    use(b);
  }
  if (j < j1) use(a);
  sink[size_t(blockIdx.x) * 256 + threadIdx.x] = acc;
}

}  // namespace

extern "C" int pkvprobe_stream_read(const void* buf, size_t bytes, void* sink, int grid,
                                    hipStream_t stream) {
  if (buf == nullptr || sink == nullptr || bytes % 16 != 0 || grid < 1 || grid > 65536)
    return -1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(buf), bytes / 16, static_cast<uint32_t*>(sink));
  return static_cast<int>(hipGetLastError());
}

extern "C" int pkvprobe_tile_read(const void* k_cache, const void* v_cache, const int* block_tables,
                                  const int* item_seq, const int* item_first, const int* item_end,
                                  int n_items, int num_kv_heads, int max_blocks_per_seq,
                                  int num_blocks, int tile_bytes, void* sink, hipStream_t stream) {
  if (k_cache == nullptr || v_cache == nullptr || block_tables == nullptr || sink == nullptr ||
      n_items < 0 || num_kv_heads < 1 || max_blocks_per_seq < 1 || num_blocks < 1 ||
      int64_t(n_items) * num_kv_heads > 0x7fffffff)
    return -1;
  if (n_items == 0) return 0;
  const dim3 grid(n_items * num_kv_heads);
  constexpr size_t kLds = 40 * 1024;          // 4 work-groups per compute unit
  const uint8_t* kc = static_cast<const uint8_t*>(k_cache);
  const uint8_t* vc = static_cast<const uint8_t*>(v_cache);
  uint32_t* out = static_cast<uint32_t*>(sink);
  switch (tile_bytes) {
    case 1024:
      hipLaunchKernelGGL(tile_read_kernel<1>, grid, dim3(256), kLds, stream, kc, vc, block_tables,
                         item_seq, item_first, item_end, num_kv_heads, max_blocks_per_seq,
                         num_blocks, out);
      break;
    case 2048:
      hipLaunchKernelGGL(tile_read_kernel<2>, grid, dim3(256), kLds, stream, kc, vc, block_tables,
                         item_seq, item_first, item_end, num_kv_heads, max_blocks_per_seq,
                         num_blocks, out);
      break;
    case 4096:
      hipLaunchKernelGGL(tile_read_kernel<4>, grid, dim3(256), kLds, stream, kc, vc, block_tables,
                         item_seq, item_first, item_end, num_kv_heads, max_blocks_per_seq,
                         num_blocks, out);
      break;
    case 8192:
      hipLaunchKernelGGL(tile_read_kernel<8>, grid, dim3(256), kLds, stream, kc, vc, block_tables,
                         item_seq, item_first, item_end, num_kv_heads, max_blocks_per_seq,
                         num_blocks, out);
      break;
    default:
      return -1;
  }
  return static_cast<int>(hipGetLastError());
}
