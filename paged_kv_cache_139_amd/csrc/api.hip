// C ABI of the library: argument checks on the host, then kernel launches on
// the caller's stream.  Declarations and the contract are in include/pagedkv.h.
#include <math.h>

#include <mutex>

#include "internal.h"
#include "pagedkv.h"

using pkv::DT;

namespace {

bool is_float_dtype(pkv_dtype t) { return t == PKV_F32 || t == PKV_F16 || t == PKV_BF16; }
bool is_known_dtype(pkv_dtype t) { return is_float_dtype(t) || t == PKV_FP8_E4M3; }
DT to_dt(pkv_dtype t) { return static_cast<DT>(static_cast<int>(t)); }

// Source / cache dtype pairs accepted by the writer and the decode.
bool pair_ok(pkv_dtype q, pkv_dtype cache) {
  if (!is_float_dtype(q)) return false;
  if (cache == q) return true;
  return cache == PKV_FP8_E4M3 && (q == PKV_F16 || q == PKV_BF16);
}

bool scale_ok(float s) { return isfinite(s) && s > 0.f; }

// Block sizes the kernels are built for, as log2 (-1: not supported).
int log2_block(int bs) { return bs == 8 ? 3 : bs == 16 ? 4 : bs == 32 ? 5 : -1; }

// head sizes the decode kernels are built for
bool head_size_ok(int32_t d) {
  switch (d) {
    case 32: case 64: case 80: case 96: case 112: case 120: case 128: case 192: case 256:
      return true;
    default:
      return false;
  }
}

// Row strides (elements) of the per-sequence tensors of a decode call.
struct RowStrides {
  long long q, out, key_new, value_new;
};

RowStrides packed_strides(int32_t H, int32_t Hk, int32_t D) {
  return {1LL * H * D, 1LL * H * D, 1LL * Hk * D, 1LL * Hk * D};
}

// A row stride of a strided call: at least the packed row (rows do not
// overlap) and a multiple of 8 elements; PKV_OK, PKV_ERR_SHAPE or
// PKV_ERR_ALIGNMENT.
pkv_status stride_ok(long long stride, long long packed) {
  if (stride < packed) return PKV_ERR_SHAPE;
  return stride % 8 == 0 ? PKV_OK : PKV_ERR_ALIGNMENT;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; }

// Partitions of P tokens that the longest possible sequence (MB blocks) needs.
int partitions(int MB, int BS, int P) { return int((1LL * MB * BS + P - 1) / P); }

// The kernels split a sequence's 16-token tiles among its partitions with
// 32-bit products (partition index x tiles): these must not overflow.
bool split_fits(int MB, int BS, int np) {
  return 1LL * np * ((1LL * MB * BS + 15) / 16) <= 0x7fffffffLL;
}

// Shared-prefix pass: blocks per prefix work-group (16 measured best on the
// parallel-sampling batch: 8 means more partials to merge, 32 too few
// work-groups), and the number of such runs a prefix of up to MB blocks needs.
constexpr int kPrefixRunBlocks = 16;
int prefix_runs(int MB) { return (MB + kPrefixRunBlocks - 1) / kPrefixRunBlocks; }

}  // namespace

extern "C" {

const char* pkv_status_string(pkv_status status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "a required pointer is NULL";
    case PKV_ERR_SHAPE: return "invalid or inconsistent size";
    case PKV_ERR_DTYPE: return "dtype combination not accepted";
    case PKV_ERR_UNSUPPORTED: return "head_size or block_size not supported";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_LAUNCH: return "kernel launch failed";
    case PKV_ERR_VALUE: return "scalar argument not finite or not positive";
    case PKV_ERR_ALIGNMENT: return "device pointer not aligned as required";
    case PKV_ERR_NO_BLOCKS: return "no free block in the pool";
    case PKV_ERR_SEQUENCE: return "unknown or already used sequence id";
    case PKV_ERR_SCRATCH: return "needs more than the no-allocation call's static scratch";
  }
  return "unknown status";
}

pkv_status reshape_and_cache(const void* key, const void* value, void* key_cache,
                             void* value_cache, const int64_t* slot_mapping, int32_t num_tokens,
                             int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                             int32_t num_blocks, pkv_dtype src_dtype, pkv_dtype cache_dtype,
                             float k_scale, float v_scale, hipStream_t stream) {
  const long long row = 1LL * num_kv_heads * head_size;
  return reshape_and_cache_strided(key, value, key_cache, value_cache, slot_mapping, num_tokens,
                                   num_kv_heads, head_size, block_size, num_blocks,
                                   num_kv_heads < 1 || head_size < 1 ? 0 : row,
                                   num_kv_heads < 1 || head_size < 1 ? 0 : row, src_dtype,
                                   cache_dtype, k_scale, v_scale, stream);
}

pkv_status reshape_and_cache_strided(const void* key, const void* value, void* key_cache,
                                     void* value_cache, const int64_t* slot_mapping,
                                     int32_t num_tokens, int32_t num_kv_heads, int32_t head_size,
                                     int32_t block_size, int32_t num_blocks,
                                     int64_t key_row_stride, int64_t value_row_stride,
                                     pkv_dtype src_dtype, pkv_dtype cache_dtype, float k_scale,
                                     float v_scale, hipStream_t stream) {
  if (num_tokens < 0 || num_kv_heads < 1 || head_size < 1 || num_blocks < 1) return PKV_ERR_SHAPE;
  if (log2_block(block_size) < 0 || head_size % 8 != 0) return PKV_ERR_UNSUPPORTED;
  if (!is_known_dtype(src_dtype) || !is_known_dtype(cache_dtype) || !pair_ok(src_dtype, cache_dtype))
    return PKV_ERR_DTYPE;
  if (cache_dtype == PKV_FP8_E4M3 && !(scale_ok(k_scale) && scale_ok(v_scale)))
    return PKV_ERR_VALUE;
  if (1LL * num_tokens * num_kv_heads * (head_size / 8) > (1LL << 38)) return PKV_ERR_SHAPE;
  const long long row = 1LL * num_kv_heads * head_size;
  for (pkv_status st : {stride_ok(key_row_stride, row), stride_ok(value_row_stride, row)})
    if (st != PKV_OK) return st;
  // the writer's work-groups cover (KV head, 256-byte chunk of a row) pairs in
  // the grid's second dimension
  const long long chunks = (1LL * head_size * pkv::dt_bytes(to_dt(src_dtype)) + 255) / 256;
  if (1LL * num_kv_heads * chunks > 65535 || num_tokens > (1 << 30)) return PKV_ERR_SHAPE;
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping) return PKV_ERR_NULL;
  if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) || !aligned16(value_cache))
    return PKV_ERR_ALIGNMENT;
  const hipError_t e = pkv::launch_reshape_and_cache(
      key, value, key_cache, value_cache, slot_mapping, num_tokens, num_kv_heads, head_size,
      num_blocks, log2_block(block_size), key_row_stride, value_row_stride, to_dt(src_dtype),
      to_dt(cache_dtype), k_scale, v_scale, stream);
  return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

size_t paged_attention_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads,
                                              int32_t head_size, int32_t max_num_blocks_per_seq,
                                              int32_t block_size, int32_t partition_size) {
  if (num_seqs < 0 || num_heads < 1 || head_size < 1 || max_num_blocks_per_seq < 1) return 0;
  if (log2_block(block_size) < 0 || max_num_blocks_per_seq > (1 << 24)) return 0;
  if (partition_size == 0) partition_size = PKV_DEFAULT_PARTITION_SIZE;
  if (partition_size < 0 || partition_size % PKV_PARTITION_QUANTUM != 0) return 0;
  const int np = partitions(max_num_blocks_per_seq, block_size, partition_size);
  if (np <= 1) return 0;
  return size_t(num_seqs) * num_heads * np * (size_t(head_size) + 2) * sizeof(float);
}

}  // extern "C"

namespace {

// paged_attention_decode, and with key_new / value_new the decode with append
pkv_status decode_call(void* out, const void* query, const void* key_new, const void* value_new,
                       const void* key_cache, const void* value_cache,
                       const int32_t* block_tables, const int32_t* context_lens,
                       int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                       int32_t head_size, int32_t block_size, int32_t max_num_blocks_per_seq,
                       int32_t num_blocks, float scale, pkv_dtype q_dtype,
                       pkv_dtype cache_dtype, float k_scale, float v_scale,
                       int32_t partition_size, void* workspace, size_t workspace_bytes,
                       hipStream_t stream, bool append, const RowStrides* strides) {
  if (num_seqs < 0 || num_heads < 1 || num_kv_heads < 1 || max_num_blocks_per_seq < 1 ||
      num_blocks < 1 || num_heads % num_kv_heads != 0)
    return PKV_ERR_SHAPE;
  if (log2_block(block_size) < 0 || !head_size_ok(head_size)) return PKV_ERR_UNSUPPORTED;
  if (!is_known_dtype(q_dtype) || !is_known_dtype(cache_dtype) || !pair_ok(q_dtype, cache_dtype))
    return PKV_ERR_DTYPE;
  if (!isfinite(scale)) return PKV_ERR_VALUE;
  if (cache_dtype == PKV_FP8_E4M3 && !(scale_ok(k_scale) && scale_ok(v_scale)))
    return PKV_ERR_VALUE;
  if (partition_size == 0) partition_size = PKV_DEFAULT_PARTITION_SIZE;
  if (partition_size < 0 || partition_size % PKV_PARTITION_QUANTUM != 0) return PKV_ERR_SHAPE;
  if (max_num_blocks_per_seq > (1 << 24)) return PKV_ERR_SHAPE;
  const int np = partitions(max_num_blocks_per_seq, block_size, partition_size);
  if (1LL * np * num_seqs * num_heads > 0x7fffffffLL) return PKV_ERR_SHAPE;
  if (!split_fits(max_num_blocks_per_seq, block_size, np)) return PKV_ERR_SHAPE;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens)
    return PKV_ERR_NULL;
  if (append && (!key_new || !value_new)) return PKV_ERR_NULL;
  const size_t need = paged_attention_decode_workspace_bytes(
      num_seqs, num_heads, head_size, max_num_blocks_per_seq, block_size, partition_size);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return PKV_ERR_WORKSPACE;

  const int g = num_heads / num_kv_heads;
  pkv::DecodeParams p;
  p.S = num_seqs;
  p.H = num_heads;
  p.Hk = num_kv_heads;
  p.g = g;
  p.MB = max_num_blocks_per_seq;
  p.NB = num_blocks;
  p.lbs = log2_block(block_size);
  p.cap = max_num_blocks_per_seq * block_size;
  p.bpp = partition_size / PKV_PARTITION_QUANTUM;
  p.np = np;
  p.np_run = np;
  p.slot0 = 0;
  p.group_starts = nullptr;
  p.group_prefix = nullptr;
  p.G = p.npp = p.ppb = p.rounds = 0;
  p.knew = p.vnew = nullptr;
  p.enc_k = p.enc_v = 1.f;
  const RowStrides packed = packed_strides(num_heads, num_kv_heads, head_size);
  const RowStrides& rs = strides ? *strides : packed;
  p.q_stride = rs.q;
  p.o_stride = rs.out;
  p.kn_stride = rs.key_new;
  p.vn_stride = rs.value_new;
  const bool fp8 = cache_dtype == PKV_FP8_E4M3;
  p.qk_scale = scale * (fp8 ? k_scale : 1.f) * 1.4426950408889634f;   // log2(e)
  p.v_scale = fp8 ? v_scale : 1.f;
  float* ws = static_cast<float*>(workspace);
  const size_t rows = size_t(num_seqs) * num_heads * np;
  p.ws_m = need ? ws : nullptr;
  p.ws_l = need ? ws + rows : nullptr;
  p.ws_acc = need ? ws + 2 * rows : nullptr;

  pkv::DecodePtrs ptr;
  ptr.out = out;
  ptr.query = query;
  ptr.kcache = static_cast<const uint8_t*>(key_cache);
  ptr.vcache = static_cast<const uint8_t*>(value_cache);
  ptr.block_tables = block_tables;
  ptr.context_lens = context_lens;

  const DT q = to_dt(q_dtype), c = to_dt(cache_dtype);
  // matrix cores for grouped heads (their kernels are built for head sizes
  // in 16-row chunks up to 128 and 192 and 256 for 16-bit caches, 64 and 128
  // for E4M3 caches, at every block size); the vector kernel for the rest
  const bool use_mfma = q != DT::F32 && g >= 2 && g <= 16 && head_size % 16 == 0 &&
                        (fp8 ? head_size == 64 || head_size == 128 : head_size <= 256);
  if (append) {
    // the decode kernel stores each new token with the block it reads
    p.knew = static_cast<const uint8_t*>(key_new);
    p.vnew = static_cast<const uint8_t*>(value_new);
    p.enc_k = fp8 ? k_scale : 1.f;
    p.enc_v = fp8 ? v_scale : 1.f;
  }
  hipError_t e = use_mfma ? pkv::launch_decode_mfma(q, c, head_size, ptr, p, stream)
                          : pkv::launch_decode_valu(q, c, head_size, ptr, p, stream);
  if (e != hipSuccess) return PKV_ERR_LAUNCH;
  if (np > 1) {
    e = pkv::launch_merge(q, head_size, ptr, p, stream);
    if (e != hipSuccess) return PKV_ERR_LAUNCH;
  }
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status paged_attention_decode(void* out, const void* query, const void* key_cache,
                                  const void* value_cache, const int32_t* block_tables,
                                  const int32_t* context_lens, int32_t num_seqs,
                                  int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                                  int32_t block_size, int32_t max_num_blocks_per_seq,
                                  int32_t num_blocks, float scale, pkv_dtype q_dtype,
                                  pkv_dtype cache_dtype, float k_scale, float v_scale,
                                  int32_t partition_size, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  return decode_call(out, query, nullptr, nullptr, key_cache, value_cache, block_tables,
                     context_lens, num_seqs, num_heads, num_kv_heads, head_size, block_size,
                     max_num_blocks_per_seq, num_blocks, scale, q_dtype, cache_dtype, k_scale,
                     v_scale, partition_size, workspace, workspace_bytes, stream, false,
                     nullptr);
}

pkv_status paged_attention_decode_append(
    void* out, const void* query, const void* key_new, const void* value_new, void* key_cache,
    void* value_cache, const int32_t* block_tables, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
    int32_t block_size, int32_t max_num_blocks_per_seq, int32_t num_blocks, float scale,
    pkv_dtype q_dtype, pkv_dtype cache_dtype, float k_scale, float v_scale,
    int32_t partition_size, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_call(out, query, key_new, value_new, key_cache, value_cache, block_tables,
                     context_lens, num_seqs, num_heads, num_kv_heads, head_size, block_size,
                     max_num_blocks_per_seq, num_blocks, scale, q_dtype, cache_dtype, k_scale,
                     v_scale, partition_size, workspace, workspace_bytes, stream, true,
                     nullptr);
}

}  // extern "C"

namespace {

// Partition results of paged_attention_decode_noalloc: one array per GPU for
// the life of the process.  In host code `scratch` names a host-side stand-in,
// not device memory; the device address comes from hipGetSymbolAddress, looked
// up once per device with that device current, and only that address is ever
// handed to a kernel.
constexpr size_t kScratchFloats = PKV_NOALLOC_SCRATCH_BYTES / sizeof(float);
static __device__ __align__(256) float scratch[kScratchFloats];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];        // device address of `scratch`, per device

// Device address of the scratch array on the current device (looked up on the
// first call there); PKV_ERR_LAUNCH if the runtime cannot provide it.
pkv_status scratch_on_current_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PKV_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return PKV_ERR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status paged_attention_decode_noalloc(void* out, const void* query, const void* key_cache,
                                          const void* value_cache, const int32_t* block_tables,
                                          const int32_t* context_lens, int32_t num_seqs,
                                          int32_t num_heads, int32_t num_kv_heads,
                                          int32_t head_size, int32_t block_size,
                                          int32_t max_num_blocks_per_seq, int32_t num_blocks,
                                          float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype,
                                          float k_scale, float v_scale, int32_t partition_size,
                                          hipStream_t stream) {
  const size_t need = paged_attention_decode_workspace_bytes(
      num_seqs, num_heads, head_size, max_num_blocks_per_seq, block_size, partition_size);
  void* ws = nullptr;
  if (need > PKV_NOALLOC_SCRATCH_BYTES) {
    // no scratch offered: decode_call reports any other argument error first,
    // else PKV_ERR_WORKSPACE, which here means the scratch is too small
    const pkv_status st = decode_call(
        out, query, nullptr, nullptr, key_cache, value_cache, block_tables, context_lens,
        num_seqs, num_heads, num_kv_heads, head_size, block_size, max_num_blocks_per_seq,
        num_blocks, scale, q_dtype, cache_dtype, k_scale, v_scale, partition_size, nullptr, 0,
        stream, false, nullptr);
    return st == PKV_ERR_WORKSPACE ? PKV_ERR_SCRATCH : st;
  }
  if (need > 0) {
    const pkv_status st = scratch_on_current_device(&ws);
    if (st != PKV_OK) return st;
  }
  return decode_call(out, query, nullptr, nullptr, key_cache, value_cache, block_tables,
                     context_lens, num_seqs, num_heads, num_kv_heads, head_size, block_size,
                     max_num_blocks_per_seq, num_blocks, scale, q_dtype, cache_dtype, k_scale,
                     v_scale, partition_size, ws, ws ? PKV_NOALLOC_SCRATCH_BYTES : 0, stream,
                     false, nullptr);
}

pkv_status paged_attention_decode_strided(
    void* out, const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t head_size, int32_t block_size,
    int32_t max_num_blocks_per_seq, int32_t num_blocks, int64_t query_row_stride,
    int64_t out_row_stride, float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype,
    float k_scale, float v_scale, int32_t partition_size, void* workspace,
    size_t workspace_bytes, hipStream_t stream) {
  if (num_heads < 1 || head_size < 1) return PKV_ERR_SHAPE;
  const RowStrides packed = packed_strides(num_heads, 1, head_size);
  const RowStrides rs{query_row_stride, out_row_stride, packed.key_new, packed.value_new};
  for (pkv_status st : {stride_ok(rs.q, packed.q), stride_ok(rs.out, packed.out)})
    if (st != PKV_OK) return st;
  if (!aligned16(query) || !aligned16(out)) return PKV_ERR_ALIGNMENT;
  return decode_call(out, query, nullptr, nullptr, key_cache, value_cache, block_tables,
                     context_lens, num_seqs, num_heads, num_kv_heads, head_size, block_size,
                     max_num_blocks_per_seq, num_blocks, scale, q_dtype, cache_dtype, k_scale,
                     v_scale, partition_size, workspace, workspace_bytes, stream, false, &rs);
}

pkv_status paged_attention_decode_append_strided(
    void* out, const void* query, const void* key_new, const void* value_new, void* key_cache,
    void* value_cache, const int32_t* block_tables, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
    int32_t block_size, int32_t max_num_blocks_per_seq, int32_t num_blocks,
    int64_t query_row_stride, int64_t key_new_row_stride, int64_t value_new_row_stride,
    int64_t out_row_stride, float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype,
    float k_scale, float v_scale, int32_t partition_size, void* workspace,
    size_t workspace_bytes, hipStream_t stream) {
  if (num_heads < 1 || num_kv_heads < 1 || head_size < 1) return PKV_ERR_SHAPE;
  const RowStrides packed = packed_strides(num_heads, num_kv_heads, head_size);
  const RowStrides rs{query_row_stride, out_row_stride, key_new_row_stride,
                      value_new_row_stride};
  for (pkv_status st : {stride_ok(rs.q, packed.q), stride_ok(rs.out, packed.out),
                        stride_ok(rs.key_new, packed.key_new),
                        stride_ok(rs.value_new, packed.value_new)})
    if (st != PKV_OK) return st;
  if (!aligned16(query) || !aligned16(out) || !aligned16(key_new) || !aligned16(value_new))
    return PKV_ERR_ALIGNMENT;
  return decode_call(out, query, key_new, value_new, key_cache, value_cache, block_tables,
                     context_lens, num_seqs, num_heads, num_kv_heads, head_size, block_size,
                     max_num_blocks_per_seq, num_blocks, scale, q_dtype, cache_dtype, k_scale,
                     v_scale, partition_size, workspace, workspace_bytes, stream, true, &rs);
}

pkv_status paged_kv_gather(void* k_out, void* v_out, const void* key_cache,
                           const void* value_cache, const int32_t* block_table_row,
                           int32_t context_len, int32_t num_kv_heads, int32_t head_size,
                           int32_t block_size, int32_t num_blocks, pkv_dtype cache_dtype,
                           hipStream_t stream) {
  if (context_len < 0 || num_kv_heads < 1 || head_size < 1 || num_blocks < 1) return PKV_ERR_SHAPE;
  if (log2_block(block_size) < 0) return PKV_ERR_UNSUPPORTED;
  if (!is_known_dtype(cache_dtype)) return PKV_ERR_DTYPE;
  if (1LL * context_len * num_kv_heads * head_size > (1LL << 38)) return PKV_ERR_SHAPE;
  if (context_len == 0) return PKV_OK;
  if (!k_out || !v_out || !key_cache || !value_cache || !block_table_row) return PKV_ERR_NULL;
  const hipError_t e = pkv::launch_gather(k_out, v_out, key_cache, value_cache, block_table_row,
                                          context_len, num_kv_heads, head_size, num_blocks,
                                          log2_block(block_size), to_dt(cache_dtype), stream);
  return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

size_t paged_attention_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_heads,
                                                            int32_t head_size,
                                                            int32_t max_num_blocks_per_seq,
                                                            int32_t block_size,
                                                            int32_t partition_size) {
  if (num_seqs < 0 || num_heads < 1 || head_size < 1 || max_num_blocks_per_seq < 1) return 0;
  if (block_size != 16 || max_num_blocks_per_seq > (1 << 24)) return 0;
  if (partition_size == 0) partition_size = PKV_DEFAULT_PARTITION_SIZE;
  if (partition_size < 0 || partition_size % PKV_PARTITION_QUANTUM != 0) return 0;
  const int slots = prefix_runs(max_num_blocks_per_seq) +
                    partitions(max_num_blocks_per_seq, block_size, partition_size);
  return size_t(num_seqs) * num_heads * slots * (size_t(head_size) + 2) * sizeof(float);
}

}  // extern "C"

namespace {

// paged_attention_decode_shared_prefix, and with key_new / value_new its
// decode with append
pkv_status shared_prefix_call(
    void* out, const void* query, const void* key_new, const void* value_new,
    const void* key_cache, const void* value_cache, const int32_t* block_tables,
    const int32_t* context_lens, const int32_t* group_starts, const int32_t* group_prefix_blocks,
    int32_t num_groups, int32_t max_group_size, int32_t num_seqs, int32_t num_heads,
    int32_t num_kv_heads, int32_t head_size, int32_t block_size, int32_t max_num_blocks_per_seq,
    int32_t num_blocks, float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype, float k_scale,
    float v_scale, int32_t partition_size, void* workspace, size_t workspace_bytes,
    hipStream_t stream, bool append) {
  if (num_seqs < 0 || num_heads < 1 || num_kv_heads < 1 || max_num_blocks_per_seq < 1 ||
      num_blocks < 1 || num_heads % num_kv_heads != 0)
    return PKV_ERR_SHAPE;
  if (num_seqs > 0 && (num_groups < 1 || num_groups > num_seqs || max_group_size < 1 ||
                       max_group_size > num_seqs))
    return PKV_ERR_SHAPE;
  if (block_size != 16 || (head_size != 64 && head_size != 128)) return PKV_ERR_UNSUPPORTED;
  const int g = num_heads / num_kv_heads;
  const bool grouped = g >= 2 && g <= 16;      // one launch on the matrix cores
  if (grouped && max_num_blocks_per_seq >= (1 << 22)) return PKV_ERR_SHAPE;   // L < 2^26
  if (append && !grouped) return PKV_ERR_UNSUPPORTED;
  if (!is_known_dtype(q_dtype) || !is_known_dtype(cache_dtype) || !pair_ok(q_dtype, cache_dtype) ||
      q_dtype == PKV_F32)
    return PKV_ERR_DTYPE;
  if (!isfinite(scale)) return PKV_ERR_VALUE;
  if (cache_dtype == PKV_FP8_E4M3 && !(scale_ok(k_scale) && scale_ok(v_scale)))
    return PKV_ERR_VALUE;
  if (partition_size == 0) partition_size = PKV_DEFAULT_PARTITION_SIZE;
  if (partition_size < 0 || partition_size % PKV_PARTITION_QUANTUM != 0) return PKV_ERR_SHAPE;
  if (max_num_blocks_per_seq > (1 << 24)) return PKV_ERR_SHAPE;
  const int np_suf = partitions(max_num_blocks_per_seq, block_size, partition_size);
  const int npp = prefix_runs(max_num_blocks_per_seq);
  const long long rounds = (1LL * max_group_size * g + 63) / 64;
  const int gm = grouped ? 16 / g : 1;                 // members per 16-row tile
  const long long gt = (1LL * max_group_size + gm - 1) / gm;
  if (1LL * np_suf * num_seqs * num_heads > 0x7fffffffLL ||
      !split_fits(max_num_blocks_per_seq, block_size, np_suf) ||
      rounds * num_groups * npp * num_kv_heads > 0x7fffffffLL ||
      ((1LL * num_groups * num_kv_heads + 7) / 8 * 8) * gt > 0x7fffffffLL)
    return PKV_ERR_SHAPE;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens ||
      !group_starts || !group_prefix_blocks)
    return PKV_ERR_NULL;
  if (append && (!key_new || !value_new)) return PKV_ERR_NULL;
  const size_t need = paged_attention_decode_shared_prefix_workspace_bytes(
      num_seqs, num_heads, head_size, max_num_blocks_per_seq, block_size, partition_size);
  if (!grouped && (workspace == nullptr || workspace_bytes < need)) return PKV_ERR_WORKSPACE;

  pkv::DecodeParams p;
  p.S = num_seqs;
  p.H = num_heads;
  p.Hk = num_kv_heads;
  p.g = g;
  p.MB = max_num_blocks_per_seq;
  p.NB = num_blocks;
  p.lbs = 4;
  p.cap = max_num_blocks_per_seq * 16;
  p.bpp = partition_size / PKV_PARTITION_QUANTUM;
  p.npp = npp;
  p.ppb = kPrefixRunBlocks;
  p.np = npp + np_suf;
  p.np_run = np_suf;
  p.slot0 = npp;
  p.group_starts = group_starts;
  p.group_prefix = group_prefix_blocks;
  p.gm = gm;
  p.gt = static_cast<int>(gt);
  p.knew = p.vnew = nullptr;
  {
    const RowStrides rs = packed_strides(num_heads, num_kv_heads, head_size);
    p.q_stride = rs.q;
    p.o_stride = rs.out;
    p.kn_stride = rs.key_new;
    p.vn_stride = rs.value_new;
  }
  p.enc_k = p.enc_v = 1.f;
  p.G = num_groups;
  p.rounds = static_cast<int>(rounds);
  const bool fp8 = cache_dtype == PKV_FP8_E4M3;
  p.qk_scale = scale * (fp8 ? k_scale : 1.f) * 1.4426950408889634f;   // log2(e)
  p.v_scale = fp8 ? v_scale : 1.f;
  if (append) {
    p.knew = static_cast<const uint8_t*>(key_new);
    p.vnew = static_cast<const uint8_t*>(value_new);
    p.enc_k = fp8 ? k_scale : 1.f;
    p.enc_v = fp8 ? v_scale : 1.f;
  }
  float* ws = static_cast<float*>(workspace);
  const size_t rows = size_t(num_seqs) * num_heads * p.np;
  p.ws_m = grouped ? nullptr : ws;
  p.ws_l = grouped ? nullptr : ws + rows;
  p.ws_acc = grouped ? nullptr : ws + 2 * rows;

  pkv::DecodePtrs ptr;
  ptr.out = out;
  ptr.query = query;
  ptr.kcache = static_cast<const uint8_t*>(key_cache);
  ptr.vcache = static_cast<const uint8_t*>(value_cache);
  ptr.block_tables = block_tables;
  ptr.context_lens = context_lens;

  const DT q = to_dt(q_dtype), c = to_dt(cache_dtype);
  if (grouped) {                           // final outputs, no workspace, no merge
    const hipError_t e = pkv::launch_decode_group(q, c, head_size, ptr, p, stream);
    return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
  }
  hipError_t e = pkv::launch_decode_prefix(q, c, head_size, ptr, p, stream);
  if (e == hipSuccess) e = pkv::launch_decode_valu(q, c, head_size, ptr, p, stream);
  if (e != hipSuccess) return PKV_ERR_LAUNCH;
  e = pkv::launch_merge(q, head_size, ptr, p, stream);
  return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

}  // namespace

extern "C" {

pkv_status paged_attention_decode_shared_prefix(
    void* out, const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens, const int32_t* group_starts,
    const int32_t* group_prefix_blocks, int32_t num_groups, int32_t max_group_size,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
    int32_t block_size, int32_t max_num_blocks_per_seq, int32_t num_blocks, float scale,
    pkv_dtype q_dtype, pkv_dtype cache_dtype, float k_scale, float v_scale,
    int32_t partition_size, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return shared_prefix_call(out, query, nullptr, nullptr, key_cache, value_cache, block_tables,
                            context_lens, group_starts, group_prefix_blocks, num_groups,
                            max_group_size, num_seqs, num_heads, num_kv_heads, head_size,
                            block_size, max_num_blocks_per_seq, num_blocks, scale, q_dtype,
                            cache_dtype, k_scale, v_scale, partition_size, workspace,
                            workspace_bytes, stream, false);
}

pkv_status paged_attention_decode_shared_prefix_append(
    void* out, const void* query, const void* key_new, const void* value_new, void* key_cache,
    void* value_cache, const int32_t* block_tables, const int32_t* context_lens,
    const int32_t* group_starts, const int32_t* group_prefix_blocks, int32_t num_groups,
    int32_t max_group_size, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
    int32_t head_size, int32_t block_size, int32_t max_num_blocks_per_seq, int32_t num_blocks,
    float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype, float k_scale, float v_scale,
    int32_t partition_size, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return shared_prefix_call(out, query, key_new, value_new, key_cache, value_cache, block_tables,
                            context_lens, group_starts, group_prefix_blocks, num_groups,
                            max_group_size, num_seqs, num_heads, num_kv_heads, head_size,
                            block_size, max_num_blocks_per_seq, num_blocks, scale, q_dtype,
                            cache_dtype, k_scale, v_scale, partition_size, workspace,
                            workspace_bytes, stream, true);
}

pkv_status copy_blocks(void* const* key_caches, void* const* value_caches, int32_t num_layers,
                       const int64_t* block_mapping, int32_t num_pairs, int32_t num_kv_heads,
                       int32_t head_size, int32_t block_size, int32_t num_blocks,
                       pkv_dtype cache_dtype, hipStream_t stream) {
  if (num_layers < 0 || num_pairs < 0 || num_kv_heads < 1 || head_size < 1 || num_blocks < 1)
    return PKV_ERR_SHAPE;
  if (log2_block(block_size) < 0) return PKV_ERR_UNSUPPORTED;
  if (!is_known_dtype(cache_dtype)) return PKV_ERR_DTYPE;
  const int64_t block_bytes =
      int64_t(num_kv_heads) * head_size * block_size * pkv::dt_bytes(to_dt(cache_dtype));
  if (block_bytes > (int64_t(1) << 40) / num_blocks) return PKV_ERR_SHAPE;
  if (int64_t(num_pairs) * pkv::copy_blocks_runs_per_block(block_bytes) > 0x7fffffffLL)
    return PKV_ERR_SHAPE;
  if (num_layers == 0 || num_pairs == 0) return PKV_OK;
  if (!key_caches || !value_caches || !block_mapping) return PKV_ERR_NULL;
  for (int i = 0; i < num_layers; ++i) {
    if (!key_caches[i] || !value_caches[i]) return PKV_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(key_caches[i]) | reinterpret_cast<uintptr_t>(value_caches[i])) &
        15)
      return PKV_ERR_ALIGNMENT;
  }
  for (int l0 = 0; l0 < num_layers; l0 += pkv::kCopyLayers) {
    const int n = num_layers - l0 < pkv::kCopyLayers ? num_layers - l0 : pkv::kCopyLayers;
    pkv::CopyLayers layers = {};
    for (int i = 0; i < n; ++i) {
      layers.k[i] = static_cast<uint8_t*>(key_caches[l0 + i]);
      layers.v[i] = static_cast<uint8_t*>(value_caches[l0 + i]);
    }
    const hipError_t e = pkv::launch_copy_blocks(layers, n, block_mapping, num_pairs, block_bytes,
                                                 num_blocks, stream);
    if (e != hipSuccess) return PKV_ERR_LAUNCH;
  }
  return PKV_OK;
}

}  // extern "C"
