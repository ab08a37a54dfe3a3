// Copy-on-write block copy: whole physical blocks (every KV head, every token
// slot) from a source id to a destination id, in the K and V caches of every
// layer ([VN] "Sharing KV Cache": a branch that appends to a block whose
// reference count exceeds one gets a fresh block holding a copy of the old
// one; [L3] "共享前缀").
//
// A block of one layer's cache is num_kv_heads * head_size * 16 elements,
// contiguous.  One work-group copies a 16 KiB run of one block of one layer,
// for K and for V: every lane moves 16 bytes per step, and the loads of a
// run are all issued before its stores.  The loads are nontemporal (each
// source byte is read once: 7% faster than cache-allocating loads), the
// stores plain (nontemporal stores were slower in a plain copy).
#include "device_common.h"
#include "internal.h"

namespace pkv {
namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopySteps = 4;                                 // 16-byte moves per lane per cache
constexpr int64_t kRunBytes = int64_t(kCopyThreads) * kCopySteps * 16;   // 16 KiB

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(CopyLayers layers,
                                                                   const int64_t* mapping,
                                                                   int64_t block_bytes,
                                                                   int64_t num_blocks,
                                                                   int runs_per_block) {
  const int pair = blockIdx.x / runs_per_block;
  const int run = blockIdx.x % runs_per_block;
  const int layer = blockIdx.y;
  const int64_t src = mapping[2 * pair];
  const int64_t dst = mapping[2 * pair + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;   // skipped pair

  const int64_t begin = run * kRunBytes + threadIdx.x * 16;
  const uint8_t* ks = layers.k[layer] + src * block_bytes;
  const uint8_t* vs = layers.v[layer] + src * block_bytes;
  uint8_t* kd = layers.k[layer] + dst * block_bytes;
  uint8_t* vd = layers.v[layer] + dst * block_bytes;
  uint4 kb[kCopySteps], vb[kCopySteps];
#pragma unroll
  for (int i = 0; i < kCopySteps; ++i) {
    const int64_t off = begin + int64_t(i) * kCopyThreads * 16;
    if (off < block_bytes) {
      kb[i] = load_nt16(ks + off);
      vb[i] = load_nt16(vs + off);
    }
  }
#pragma unroll
  for (int i = 0; i < kCopySteps; ++i) {
    const int64_t off = begin + int64_t(i) * kCopyThreads * 16;
    if (off < block_bytes) {
      *reinterpret_cast<uint4*>(kd + off) = kb[i];
      *reinterpret_cast<uint4*>(vd + off) = vb[i];
    }
  }
}

}  // namespace

hipError_t launch_copy_blocks(const CopyLayers& layers, int num_layers, const int64_t* mapping,
                              int num_pairs, int64_t block_bytes, int64_t num_blocks,
                              hipStream_t stream) {
  const int runs = static_cast<int>((block_bytes + kRunBytes - 1) / kRunBytes);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(unsigned(num_pairs) * unsigned(runs), num_layers),
                     dim3(kCopyThreads), 0, stream, layers, mapping, block_bytes, num_blocks, runs);
  return hipGetLastError();
}

int64_t copy_blocks_runs_per_block(int64_t block_bytes) {
  return (block_bytes + kRunBytes - 1) / kRunBytes;
}

}  // namespace pkv
