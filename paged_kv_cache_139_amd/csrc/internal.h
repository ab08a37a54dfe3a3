// Declarations shared between the C-ABI layer (api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

enum class DT : int { F32 = 0, F16 = 1, BF16 = 2, FP8 = 3 };

constexpr int kBlockSize = 16;

inline int dt_bytes(DT t) {
  switch (t) {
    case DT::F32: return 4;
    case DT::F16: return 2;
    case DT::BF16: return 2;
    default: return 1;
  }
}

// Everything a decode launch needs besides the data pointers.
struct DecodeParams {
  int S, H, Hk, g, MB, NB;
  int lbs;        // log2(BLOCK_SIZE)
  int cap;        // MB * BLOCK_SIZE: most tokens a sequence can hold
  int bpp;        // 16-token tiles per partition (blocks, when BLOCK_SIZE is 16)
  int np;         // workspace slots per (sequence, head)
  int np_run;     // partitions the decode kernel's grid covers (max over the batch)
  int slot0;      // workspace slot of the decode kernel's partition 0
  float qk_scale; // scale * k_scale * log2(e): logits are kept in base-2 units
  float v_scale;
  float* ws_m;    // [S, H, np] running max (base 2)
  float* ws_l;    // [S, H, np] sum of exponentials
  float* ws_acc;  // [S, H, np, D] un-normalised weighted sum of values
  // Shared-prefix batches (group_starts != nullptr): the sequences of group
  // k are group_starts[k] .. group_starts[k + 1] - 1 and share their first
  // group_prefix[k] blocks.  The prefix pass fills slots 0 .. npp - 1 (runs
  // of ppb blocks, up to 4 x 16 query rows per work-group, `rounds` row
  // rounds); the decode kernels then cover each sequence's remaining blocks
  // from slot npp on, and the merge combines all np slots.
  const int32_t* group_starts;
  const int32_t* group_prefix;
  int G, npp, ppb, rounds;
  // Shared-prefix batches on the matrix cores (decode_group_kernel): a
  // work-group takes one 16-row tile of gm members x g query heads of one KV
  // head; gt tiles cover the largest group.
  int gm, gt;
  // Decode with append (plain batches, knew != nullptr): each sequence's new
  // token, rows [S, Hk, D] in the query dtype, is stored at logical position
  // context_len - 1 (as the writer would: a bit copy, or E4M3 of x / enc_k,
  // x / enc_v) by the wave that reads that block, which also attends over it.
  const uint8_t* knew;
  const uint8_t* vnew;
  float enc_k, enc_v;
  // Row strides in elements: sequence s's query row starts at element
  // s * q_stride, its output row at s * o_stride and its new key / value
  // rows at s * kn_stride / s * vn_stride (heads and elements contiguous
  // within a row; H * D and Hk * D for packed tensors).
  long long q_stride, o_stride, kn_stride, vn_stride;
};

struct DecodePtrs {
  void* out;
  const void* query;
  const uint8_t* kcache;
  const uint8_t* vcache;
  const int32_t* block_tables;
  const int32_t* context_lens;
};

hipError_t launch_decode_valu(DT q, DT c, int D, const DecodePtrs& ptr, const DecodeParams& p,
                              hipStream_t stream);
hipError_t launch_decode_mfma(DT q, DT c, int D, const DecodePtrs& ptr, const DecodeParams& p,
                              hipStream_t stream);
hipError_t launch_decode_prefix(DT q, DT c, int D, const DecodePtrs& ptr, const DecodeParams& p,
                                hipStream_t stream);
// a shared-prefix batch in one launch with no partial results (2 <= g <= 16)
hipError_t launch_decode_group(DT q, DT c, int D, const DecodePtrs& ptr, const DecodeParams& p,
                               hipStream_t stream);
hipError_t launch_merge(DT q, int D, const DecodePtrs& ptr, const DecodeParams& p,
                        hipStream_t stream);

// key / value rows of token t start at elements t * kst / t * vst
hipError_t launch_reshape_and_cache(const void* key, const void* value, void* kc, void* vc,
                                    const int64_t* slots, int T, int Hk, int D, int NB, int lbs,
                                    long long kst, long long vst, DT src, DT cache,
                                    float k_scale, float v_scale, hipStream_t stream);
// Cache base pointers of up to kCopyLayers layers, passed by value.
constexpr int kCopyLayers = 32;
struct CopyLayers {
  uint8_t* k[kCopyLayers];
  uint8_t* v[kCopyLayers];
};
hipError_t launch_copy_blocks(const CopyLayers& layers, int num_layers, const int64_t* mapping,
                              int num_pairs, int64_t block_bytes, int64_t num_blocks,
                              hipStream_t stream);
int64_t copy_blocks_runs_per_block(int64_t block_bytes);

hipError_t launch_gather(void* k_out, void* v_out, const void* kc, const void* vc,
                         const int32_t* table, int L, int Hk, int D, int NB, int lbs, DT cache,
                         hipStream_t stream);

}  // namespace pkv
