// Paged decode attention for grouped-query heads on the CDNA4 matrix cores.
//
// When g = num_heads / num_kv_heads query heads read the same KV head, one
// wavefront takes all g of them for one (partition, sequence, KV head): each
// K/V tile is read from HBM once and scores / weighted sums become real
// [16 x 16 x 16] contractions (v_mfma_f32_16x16x16 on f16 or bf16; g <= 16
// rows of the 16 are used).  Block walk and partitioning as in the VALU
// kernel ([L3] "注意力计算的'分页'实现"; [TGI] §4.1, §4.3).
//
// MFMA operand layouts (lane = 16 * kq + n, item i = 0..3):
//   A[m][k]: m = n, k = 4 kq + i;  B[k][n]: k = 4 kq + i, n = n;
//   C[m][n]: m = 4 kq + i, n = n.
//
// A 16-row chunk of a tile, K[d][t] (token fastest, [TGI] §4.2), loads
// naturally as A[m = d][k = t].  Scores need the contraction over d, so each
// chunk is first transposed by an MFMA against the identity (exact: every
// product is x*1 or x*0, tail tokens are zeroed beforehand), which leaves
// K[d = 4 kq + i][t = n] in C layout = A layout of S^T = K^T Q^T.  The result
// S^T lands as S[h = n][t = 4 kq + i]: every lane owns one head's running max
// and sum.  The weighted sum is computed transposed, O^T = V P^T: V's natural
// load is the A operand and the probabilities are already in B layout, and
// O^T[d = 4 kq + i][h = n] keeps each lane on its own head, so rescaling by
// exp(m_old - m_new) needs no data movement.  Probabilities are split into a
// high and a low 16-bit part (two MFMAs) so that the weighted sum keeps about
// 16 bits of each weight before float32 accumulation.
#include <type_traits>

#include "device_common.h"

namespace pkv {
namespace {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <DT Q> struct Mfma;
template <> struct Mfma<DT::F16> {
  using vec = half4_t;
  static __device__ __forceinline__ float4_t run(vec a, vec b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ short bits(float x) {
    return __builtin_bit_cast(short, static_cast<_Float16>(x));
  }
  static __device__ __forceinline__ float value(short b) {
    return static_cast<float>(__builtin_bit_cast(_Float16, b));
  }
  static __device__ __forceinline__ vec from_bits(short4_t v) {
    return __builtin_bit_cast(vec, v);
  }
  // 4 E4M3 codes -> 4 f16, two per instruction (exact: every E4M3 value is an
  // f16 value, and a scale of 1 leaves it unchanged)
  static __device__ __forceinline__ short4_t fp8x4(uint32_t w) {
    const auto lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
    const auto hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
    return __builtin_bit_cast(short4_t, u32x2_t{__builtin_bit_cast(uint32_t, lo),
                                                __builtin_bit_cast(uint32_t, hi)});
  }
};
template <> struct Mfma<DT::BF16> {
  using vec = short4_t;
  static __device__ __forceinline__ float4_t run(vec a, vec b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ short bits(float x) {
    return __builtin_bit_cast(short, static_cast<__bf16>(x));
  }
  static __device__ __forceinline__ float value(short b) {
    return __uint_as_float(static_cast<uint32_t>(static_cast<uint16_t>(b)) << 16);
  }
  static __device__ __forceinline__ vec from_bits(short4_t v) { return v; }
  // 4 E4M3 codes -> 4 bf16, two per instruction (exact: every E4M3 value is a
  // bf16 value, and a scale of 1 leaves it unchanged)
  static __device__ __forceinline__ short4_t fp8x4(uint32_t w) {
    const auto lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
    const auto hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
    return __builtin_bit_cast(short4_t, u32x2_t{__builtin_bit_cast(uint32_t, lo),
                                                __builtin_bit_cast(uint32_t, hi)});
  }
};

// One lane's 4 tokens of one row of a 16-row chunk, as loaded (raw bits).
template <DT CDT> struct RawChunk { using type = short4_t; };
template <> struct RawChunk<DT::FP8> { using type = uint32_t; };

// FP8 tiles are staged through LDS instead: each lane's 4-byte operand load
// moves only 256 bytes per instruction, and those loads measured ~30% slower
// than copying the tile with the direct global->LDS load (16 bytes per lane,
// 1 KiB per instruction) and reading the operands back from LDS.  The copy
// is an exact image of the tile; a stage holds K, then V.  The operand reads
// below are inline assembly whose wait for their data is part of the same
// statement, so no result is used before it has arrived (and the compiler,
// which does not see them as LDS reads, adds no wait for the copies still in
// flight into the other stages).
__device__ __forceinline__ void split_qwords(u32x4_t r, short4_t& a, short4_t& b) {
  a = __builtin_bit_cast(short4_t, u32x2_t{r.x, r.y});
  b = __builtin_bit_cast(short4_t, u32x2_t{r.z, r.w});
}

// Transposed K with the natural V: the transposing LDS reads hand each lane
// K^T operands directly.  A ds_read_b64_tr_b16 by a 16-lane group returns,
// to lane j, column j of the 4 x 16 matrix of 16-bit elements that the 16
// lanes' 8-byte reads form in lane order (row r = lanes 4r .. 4r + 3);
// ds_read_b64_tr_b8 does the same with an 8 x 16 matrix of bytes (row r =
// lanes 2r, 2r + 1).  Lane (kq, n) therefore points its read at the row
// segment that lane n of the output needs: for 16-bit K at K[d][4 (n % 4)]
// with d = 16 c + 4 kq + n / 4, so that lane n receives K[16 c + 4 kq + i][n]
// for i = 0..3 -- the A operand of S^T = K^T Q^T, with no data crossing
// tokens, so a token's NaN stays in its own score.  For FP8, one read covers
// chunks c and c + 1: row i < 4 is K[16 c + 4 kq + i], row i >= 4 is
// K[16 (c + 1) + 4 kq + i - 4].  V is read in its natural layout: chunk c at
// 16 * 16 * E * c bytes, so ds_read2st64 pairs with offsets in chunk strides
// (64 dwords for FP8, 64 qwords for 16-bit caches).
template <DT CDT, int NC> struct StagedKtV;
template <> struct StagedKtV<DT::FP8, 8> {
  static __device__ __forceinline__ void read(uint32_t kt, uint32_t va, u32x2_t (&k)[4],
                                              uint32_t (&v)[8]) {
    u32x2_t v0, v1, v2, v3;
    asm volatile(
        "ds_read_b64_tr_b8 %0, %8 offset:0\n\t"
        "ds_read_b64_tr_b8 %1, %8 offset:512\n\t"
        "ds_read_b64_tr_b8 %2, %8 offset:1024\n\t"
        "ds_read_b64_tr_b8 %3, %8 offset:1536\n\t"
        "ds_read2st64_b32 %4, %9 offset0:0 offset1:1\n\t"
        "ds_read2st64_b32 %5, %9 offset0:2 offset1:3\n\t"
        "ds_read2st64_b32 %6, %9 offset0:4 offset1:5\n\t"
        "ds_read2st64_b32 %7, %9 offset0:6 offset1:7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(v0), "=&v"(v1), "=&v"(v2),
          "=&v"(v3)
        : "v"(kt), "v"(va)
        : "memory");
    const u32x2_t vv[4] = {v0, v1, v2, v3};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = vv[i].x;
      v[2 * i + 1] = vv[i].y;
    }
  }
};
template <> struct StagedKtV<DT::FP8, 4> {
  static __device__ __forceinline__ void read(uint32_t kt, uint32_t va, u32x2_t (&k)[2],
                                              uint32_t (&v)[4]) {
    u32x2_t v0, v1;
    asm volatile(
        "ds_read_b64_tr_b8 %0, %4 offset:0\n\t"
        "ds_read_b64_tr_b8 %1, %4 offset:512\n\t"
        "ds_read2st64_b32 %2, %5 offset0:0 offset1:1\n\t"
        "ds_read2st64_b32 %3, %5 offset0:2 offset1:3\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k[0]), "=&v"(k[1]), "=&v"(v0), "=&v"(v1)
        : "v"(kt), "v"(va)
        : "memory");
    v[0] = v0.x;
    v[1] = v0.y;
    v[2] = v1.x;
    v[3] = v1.y;
  }
};
template <> struct StagedKtV<DT::BF16, 8> {
  static __device__ __forceinline__ void read(uint32_t kt, uint32_t va, u32x2_t (&k)[8],
                                              short4_t (&v)[8]) {
    u32x4_t v0, v1, v2, v3;
    asm volatile(
        "ds_read_b64_tr_b16 %0, %12 offset:0\n\t"
        "ds_read_b64_tr_b16 %1, %12 offset:512\n\t"
        "ds_read_b64_tr_b16 %2, %12 offset:1024\n\t"
        "ds_read_b64_tr_b16 %3, %12 offset:1536\n\t"
        "ds_read_b64_tr_b16 %4, %12 offset:2048\n\t"
        "ds_read_b64_tr_b16 %5, %12 offset:2560\n\t"
        "ds_read_b64_tr_b16 %6, %12 offset:3072\n\t"
        "ds_read_b64_tr_b16 %7, %12 offset:3584\n\t"
        "ds_read2st64_b64 %8, %13 offset0:0 offset1:1\n\t"
        "ds_read2st64_b64 %9, %13 offset0:2 offset1:3\n\t"
        "ds_read2st64_b64 %10, %13 offset0:4 offset1:5\n\t"
        "ds_read2st64_b64 %11, %13 offset0:6 offset1:7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(k[4]), "=&v"(k[5]),
          "=&v"(k[6]), "=&v"(k[7]), "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3)
        : "v"(kt), "v"(va)
        : "memory");
    split_qwords(v0, v[0], v[1]);
    split_qwords(v1, v[2], v[3]);
    split_qwords(v2, v[4], v[5]);
    split_qwords(v3, v[6], v[7]);
  }
};
template <> struct StagedKtV<DT::BF16, 4> {
  static __device__ __forceinline__ void read(uint32_t kt, uint32_t va, u32x2_t (&k)[4],
                                              short4_t (&v)[4]) {
    u32x4_t v0, v1;
    asm volatile(
        "ds_read_b64_tr_b16 %0, %6 offset:0\n\t"
        "ds_read_b64_tr_b16 %1, %6 offset:512\n\t"
        "ds_read_b64_tr_b16 %2, %6 offset:1024\n\t"
        "ds_read_b64_tr_b16 %3, %6 offset:1536\n\t"
        "ds_read2st64_b64 %4, %7 offset0:0 offset1:1\n\t"
        "ds_read2st64_b64 %5, %7 offset0:2 offset1:3\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(v0), "=&v"(v1)
        : "v"(kt), "v"(va)
        : "memory");
    split_qwords(v0, v[0], v[1]);
    split_qwords(v1, v[2], v[3]);
  }
};
template <int NC> struct StagedKtV<DT::F16, NC> : StagedKtV<DT::BF16, NC> {};

// The K^T operands alone from a staged 16-bit K tile (V in registers).
template <int NC> struct StagedKt16;
template <> struct StagedKt16<8> {
  static __device__ __forceinline__ void read(uint32_t kt, u32x2_t (&k)[8]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:0\n\t"
        "ds_read_b64_tr_b16 %1, %8 offset:512\n\t"
        "ds_read_b64_tr_b16 %2, %8 offset:1024\n\t"
        "ds_read_b64_tr_b16 %3, %8 offset:1536\n\t"
        "ds_read_b64_tr_b16 %4, %8 offset:2048\n\t"
        "ds_read_b64_tr_b16 %5, %8 offset:2560\n\t"
        "ds_read_b64_tr_b16 %6, %8 offset:3072\n\t"
        "ds_read_b64_tr_b16 %7, %8 offset:3584\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(k[4]), "=&v"(k[5]),
          "=&v"(k[6]), "=&v"(k[7])
        : "v"(kt)
        : "memory");
  }
};
template <> struct StagedKt16<2> {
  static __device__ __forceinline__ void read(uint32_t kt, u32x2_t (&k)[2]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %2 offset:0\n\t"
        "ds_read_b64_tr_b16 %1, %2 offset:512\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k[0]), "=&v"(k[1])
        : "v"(kt)
        : "memory");
  }
};
template <> struct StagedKt16<4> {
  static __device__ __forceinline__ void read(uint32_t kt, u32x2_t (&k)[4]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4 offset:0\n\t"
        "ds_read_b64_tr_b16 %1, %4 offset:512\n\t"
        "ds_read_b64_tr_b16 %2, %4 offset:1024\n\t"
        "ds_read_b64_tr_b16 %3, %4 offset:1536\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3])
        : "v"(kt)
        : "memory");
  }
};

// E4M3 steps at BLOCK_SIZE 8: the LDS image holds the step's two block tiles
// one after the other, [first: D rows x 8 bytes][second: D rows x 8 bytes]
// (each a contiguous copy of its cache tile).  The transposing K reads then
// cover two chunks (32 rows) per 256 bytes of a tile, and a lane's V bytes of
// chunk c lie 128 c bytes into its block's tile.
template <int NC> struct StagedKtV8;
template <> struct StagedKtV8<8> {
  static __device__ __forceinline__ void read(uint32_t kt, uint32_t va, u32x2_t (&k)[4],
                                              uint32_t (&v)[8]) {
    u32x2_t v0, v1, v2, v3;
    asm volatile(
        "ds_read_b64_tr_b8 %0, %8 offset:0\n\t"
        "ds_read_b64_tr_b8 %1, %8 offset:256\n\t"
        "ds_read_b64_tr_b8 %2, %8 offset:512\n\t"
        "ds_read_b64_tr_b8 %3, %8 offset:768\n\t"
        "ds_read2_b32 %4, %9 offset0:0 offset1:32\n\t"
        "ds_read2_b32 %5, %9 offset0:64 offset1:96\n\t"
        "ds_read2_b32 %6, %9 offset0:128 offset1:160\n\t"
        "ds_read2_b32 %7, %9 offset0:192 offset1:224\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(v0), "=&v"(v1), "=&v"(v2),
          "=&v"(v3)
        : "v"(kt), "v"(va)
        : "memory");
    const u32x2_t vv[4] = {v0, v1, v2, v3};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = vv[i].x;
      v[2 * i + 1] = vv[i].y;
    }
  }
};
template <> struct StagedKtV8<4> {
  static __device__ __forceinline__ void read(uint32_t kt, uint32_t va, u32x2_t (&k)[2],
                                              uint32_t (&v)[4]) {
    u32x2_t v0, v1;
    asm volatile(
        "ds_read_b64_tr_b8 %0, %4 offset:0\n\t"
        "ds_read_b64_tr_b8 %1, %4 offset:256\n\t"
        "ds_read2_b32 %2, %5 offset0:0 offset1:32\n\t"
        "ds_read2_b32 %3, %5 offset0:64 offset1:96\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k[0]), "=&v"(k[1]), "=&v"(v0), "=&v"(v1)
        : "v"(kt), "v"(va)
        : "memory");
    v[0] = v0.x;
    v[1] = v0.y;
    v[2] = v1.x;
    v[3] = v1.y;
  }
};

// The same reads from the image of a whole 32-token E4M3 block ([D][32]
// bytes): rows and chunks are twice as far apart; the lane addresses select
// the 16-token half (see kt_lane_offset32).
template <int NC> struct StagedKtV32;
template <> struct StagedKtV32<8> {
  static __device__ __forceinline__ void read(uint32_t kt, uint32_t va, u32x2_t (&k)[4],
                                              uint32_t (&v)[8]) {
    u32x2_t v0, v1, v2, v3;
    asm volatile(
        "ds_read_b64_tr_b8 %0, %8 offset:0\n\t"
        "ds_read_b64_tr_b8 %1, %8 offset:1024\n\t"
        "ds_read_b64_tr_b8 %2, %8 offset:2048\n\t"
        "ds_read_b64_tr_b8 %3, %8 offset:3072\n\t"
        "ds_read2st64_b32 %4, %9 offset0:0 offset1:2\n\t"
        "ds_read2st64_b32 %5, %9 offset0:4 offset1:6\n\t"
        "ds_read2st64_b32 %6, %9 offset0:8 offset1:10\n\t"
        "ds_read2st64_b32 %7, %9 offset0:12 offset1:14\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(v0), "=&v"(v1), "=&v"(v2),
          "=&v"(v3)
        : "v"(kt), "v"(va)
        : "memory");
    const u32x2_t vv[4] = {v0, v1, v2, v3};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = vv[i].x;
      v[2 * i + 1] = vv[i].y;
    }
  }
  static __device__ __forceinline__ void read_k(uint32_t kt, u32x2_t (&k)[4]) {
    asm volatile(
        "ds_read_b64_tr_b8 %0, %4 offset:0\n\t"
        "ds_read_b64_tr_b8 %1, %4 offset:1024\n\t"
        "ds_read_b64_tr_b8 %2, %4 offset:2048\n\t"
        "ds_read_b64_tr_b8 %3, %4 offset:3072\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3])
        : "v"(kt)
        : "memory");
  }
  static __device__ __forceinline__ void read_v(uint32_t va, uint32_t (&v)[8]) {
    u32x2_t v0, v1, v2, v3;
    asm volatile(
        "ds_read2st64_b32 %0, %4 offset0:0 offset1:2\n\t"
        "ds_read2st64_b32 %1, %4 offset0:4 offset1:6\n\t"
        "ds_read2st64_b32 %2, %4 offset0:8 offset1:10\n\t"
        "ds_read2st64_b32 %3, %4 offset0:12 offset1:14\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3)
        : "v"(va)
        : "memory");
    const u32x2_t vv[4] = {v0, v1, v2, v3};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = vv[i].x;
      v[2 * i + 1] = vv[i].y;
    }
  }
};
template <> struct StagedKtV32<4> {
  static __device__ __forceinline__ void read(uint32_t kt, uint32_t va, u32x2_t (&k)[2],
                                              uint32_t (&v)[4]) {
    read_k(kt, k);
    read_v(va, v);
  }
  static __device__ __forceinline__ void read_k(uint32_t kt, u32x2_t (&k)[2]) {
    asm volatile(
        "ds_read_b64_tr_b8 %0, %2 offset:0\n\t"
        "ds_read_b64_tr_b8 %1, %2 offset:1024\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k[0]), "=&v"(k[1])
        : "v"(kt)
        : "memory");
  }
  static __device__ __forceinline__ void read_v(uint32_t va, uint32_t (&v)[4]) {
    u32x2_t v0, v1;
    asm volatile(
        "ds_read2st64_b32 %0, %2 offset0:0 offset1:2\n\t"
        "ds_read2st64_b32 %1, %2 offset0:4 offset1:6\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v0), "=&v"(v1)
        : "v"(va)
        : "memory");
    v[0] = v0.x;
    v[1] = v0.y;
    v[2] = v1.x;
    v[3] = v1.y;
  }
};

// K^T operands of a 32-token tile of a 16-bit cache from its LDS image, NC
// chunks of 16 rows CH bytes apart (the block size's row bytes x 16); the
// lane addresses select the tokens (see mfma_walk).
template <int NC, int CH> struct StagedKt16T;
template <int CH> struct StagedKt16T<8, CH> {
  static __device__ __forceinline__ void read_k(uint32_t kt, u32x2_t (&k)[8]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:0\n\t"
        "ds_read_b64_tr_b16 %1, %8 offset:%9\n\t"
        "ds_read_b64_tr_b16 %2, %8 offset:%10\n\t"
        "ds_read_b64_tr_b16 %3, %8 offset:%11\n\t"
        "ds_read_b64_tr_b16 %4, %8 offset:%12\n\t"
        "ds_read_b64_tr_b16 %5, %8 offset:%13\n\t"
        "ds_read_b64_tr_b16 %6, %8 offset:%14\n\t"
        "ds_read_b64_tr_b16 %7, %8 offset:%15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(k[4]), "=&v"(k[5]),
          "=&v"(k[6]), "=&v"(k[7])
        : "v"(kt), "n"(CH), "n"(2 * CH), "n"(3 * CH), "n"(4 * CH), "n"(5 * CH), "n"(6 * CH),
          "n"(7 * CH)
        : "memory");
  }
};
template <int CH> struct StagedKt16T<4, CH> {
  static __device__ __forceinline__ void read_k(uint32_t kt, u32x2_t (&k)[4]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4 offset:0\n\t"
        "ds_read_b64_tr_b16 %1, %4 offset:%5\n\t"
        "ds_read_b64_tr_b16 %2, %4 offset:%6\n\t"
        "ds_read_b64_tr_b16 %3, %4 offset:%7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3])
        : "v"(kt), "n"(CH), "n"(2 * CH), "n"(3 * CH)
        : "memory");
  }
};
template <int CH> struct StagedKt16T<2, CH> {
  static __device__ __forceinline__ void read_k(uint32_t kt, u32x2_t (&k)[2]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %2 offset:0\n\t"
        "ds_read_b64_tr_b16 %1, %2 offset:%3\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k[0]), "=&v"(k[1])
        : "v"(kt), "n"(CH)
        : "memory");
  }
};
template <int CH> struct StagedKt16T<5, CH> {
  static __device__ __forceinline__ void read_k(uint32_t kt, u32x2_t (&k)[5]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %5 offset:0\n\t"
        "ds_read_b64_tr_b16 %1, %5 offset:%6\n\t"
        "ds_read_b64_tr_b16 %2, %5 offset:%7\n\t"
        "ds_read_b64_tr_b16 %3, %5 offset:%8\n\t"
        "ds_read_b64_tr_b16 %4, %5 offset:%9\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(k[4])
        : "v"(kt), "n"(CH), "n"(2 * CH), "n"(3 * CH), "n"(4 * CH)
        : "memory");
  }
};
template <int CH> struct StagedKt16T<6, CH> {
  static __device__ __forceinline__ void read_k(uint32_t kt, u32x2_t (&k)[6]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %6 offset:0\n\t"
        "ds_read_b64_tr_b16 %1, %6 offset:%7\n\t"
        "ds_read_b64_tr_b16 %2, %6 offset:%8\n\t"
        "ds_read_b64_tr_b16 %3, %6 offset:%9\n\t"
        "ds_read_b64_tr_b16 %4, %6 offset:%10\n\t"
        "ds_read_b64_tr_b16 %5, %6 offset:%11\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(k[4]), "=&v"(k[5])
        : "v"(kt), "n"(CH), "n"(2 * CH), "n"(3 * CH), "n"(4 * CH), "n"(5 * CH)
        : "memory");
  }
};
template <int CH> struct StagedKt16T<7, CH> {
  static __device__ __forceinline__ void read_k(uint32_t kt, u32x2_t (&k)[7]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %7 offset:0\n\t"
        "ds_read_b64_tr_b16 %1, %7 offset:%8\n\t"
        "ds_read_b64_tr_b16 %2, %7 offset:%9\n\t"
        "ds_read_b64_tr_b16 %3, %7 offset:%10\n\t"
        "ds_read_b64_tr_b16 %4, %7 offset:%11\n\t"
        "ds_read_b64_tr_b16 %5, %7 offset:%12\n\t"
        "ds_read_b64_tr_b16 %6, %7 offset:%13\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(k[4]), "=&v"(k[5]),
          "=&v"(k[6])
        : "v"(kt), "n"(CH), "n"(2 * CH), "n"(3 * CH), "n"(4 * CH), "n"(5 * CH), "n"(6 * CH)
        : "memory");
  }
};

// Lane byte offsets of the transposing K read and of the V reads in an E4M3
// stage at BLOCK_SIZE 8 (see StagedKtV8; D rows per block tile): the lane's
// K segment (row d, tokens 8 (n & 1) ..) lies in the first or the second
// tile, its V tokens 4 kq .. 4 kq + 3 of row n in the tile of kq >> 1.
__device__ __forceinline__ uint32_t kt_lane_offset8(int kq, int n, int D) {
  const int i = n >> 1;
  const int d = i < 4 ? 4 * kq + i : 16 + 4 * kq + (i - 4);
  return uint32_t(d * 8 + (n & 1) * D * 8);
}
__device__ __forceinline__ uint32_t v_lane_offset8(int kq, int n, int D) {
  return uint32_t((kq >> 1) * D * 8 + n * 8 + 4 * (kq & 1));
}

// Lane byte offset of the transposing K read in a whole-block E4M3 image
// (StagedKtV32): as kt_lane_offset's, with 32-byte rows; the second 16-token
// half adds 16.
__device__ __forceinline__ uint32_t kt_lane_offset32(int kq, int n) {
  const int i = n >> 1;
  const int d = i < 4 ? 4 * kq + i : 16 + 4 * kq + (i - 4);
  return uint32_t(d * 32 + 8 * (n & 1));
}

// Lane byte offset of the transposing K read within a stage (see StagedKtV).
template <DT CDT>
__device__ __forceinline__ uint32_t kt_lane_offset(int kq, int n) {
  if constexpr (CDT == DT::FP8) {
    const int i = n >> 1;                                 // output row of this lane's segment
    const int d = i < 4 ? 4 * kq + i : 16 + 4 * kq + (i - 4);
    return uint32_t(d * kBlockSize + 8 * (n & 1));
  } else {
    const int d = 4 * kq + (n >> 2);
    return uint32_t((d * kBlockSize + 4 * (n & 3)) * 2);
  }
}

// K^T operands of the NC chunks from what StagedKtV returned.
template <DT QDT, DT CDT, int NC>
__device__ __forceinline__ void kt_operands(const u32x2_t (&k)[CDT == DT::FP8 ? NC / 2 : NC],
                                            short4_t (&kt)[NC]) {
  if constexpr (CDT == DT::FP8) {
#pragma unroll
    for (int c = 0; c < NC / 2; ++c) {
      kt[2 * c] = Mfma<QDT>::fp8x4(k[c].x);
      kt[2 * c + 1] = Mfma<QDT>::fp8x4(k[c].y);
    }
  } else {
#pragma unroll
    for (int c = 0; c < NC; ++c) kt[c] = __builtin_bit_cast(short4_t, k[c]);
  }
}

// Wait until at most N vector-memory operations of this wave are outstanding
// (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Cache policy of the decode walk's direct global->LDS tile copies:
// nontemporal.  On the FP8 batch with lognormal lengths they measured 13%
// faster than cache-allocating copies (98.9 -> 85.6 us), and on FP8
// shared-prefix batches through the plain call (8 samples reading each prefix
// block at about the same time) they cost nothing (50.0 us either way).  The
// shared-prefix pass keeps cache-allocating copies: nontemporal ones measured
// 3% slower on the whole shared-prefix call.
constexpr int kDmaNontemporal = 2;
constexpr int kDmaPrefix = 0;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) uint8_t lds_u8_t;

__device__ __forceinline__ uint32_t lds_address(const uint8_t* p) {
  return static_cast<uint32_t>(reinterpret_cast<size_t>((const lds_u8_t*)(p)));
}

// Plain (cache-allocating) loads: when sequences share prefix blocks (parallel
// sampling) the other samples find those tiles in L2 / Infinity Cache;
// nontemporal loads measured 20% slower on the shared-prefix batch.
template <DT CDT>
__device__ __forceinline__ typename RawChunk<CDT>::type load_raw(const uint8_t* p) {
  return *reinterpret_cast<const typename RawChunk<CDT>::type*>(p);
}

// raw bits -> 16-bit MFMA operand bits (FP8 codes are decoded exactly)
template <DT QDT, DT CDT>
__device__ __forceinline__ short4_t to_operand(typename RawChunk<CDT>::type r) {
  if constexpr (CDT == DT::FP8) {
    return Mfma<QDT>::fp8x4(r);
  } else {
    return r;
  }
}

// LDS of the decode walk: per wave, FP8 caches keep two K/V stages (two
// stages at 4 waves per SIMD measured faster than three or four stages at
// lower occupancy); after the walk the same bytes hold the wave's partial
// O[h][d] for the combine.
template <DT CDT, int D>
struct MfmaLds {
  static constexpr size_t kTileBytes = size_t(D) * kBlockSize * Elem<CDT>::bytes;
  static constexpr int kStages = 2;
  static constexpr int kCombine = 16 * D * 4;
  static constexpr int kStage = CDT == DT::FP8 ? kStages * 2 * int(kTileBytes) : 0;
  static constexpr int kWave = kStage > kCombine ? kStage : kCombine;
  static constexpr int kBytes = kWaves * kWave;
};

// Cache block sizes of the walk.  The walk steps through a sequence 16 tokens
// at a time (a "step"): at BLOCK_SIZE 16 a step is a block, at 8 two blocks
// (the second may be missing).  K and V chunks are 16 rows x 16 tokens either
// way: lane (kq, n) holds tokens 4 kq .. 4 kq + 3 of row 16 c + n, which at
// BLOCK_SIZE 8 lie in the step's first block for kq < 2 and in its second for
// kq >= 2.  E4M3 steps are copied into an LDS image [D][16]: 1 KiB per
// instruction from one contiguous tile at 16, 4 bytes per lane at 8 (each
// 16-byte image row takes 8 bytes from each block).  At 32 the E4M3 walk
// takes whole blocks instead, and the 16-bit walk (head sizes up to 128)
// takes 32-token tiles at every block size (see mfma_walk); the 16-token
// steps of 16-bit caches remain for head sizes 192 and 256.
template <int BS> struct Steps {
  static_assert(BS == 8 || BS == 16 || BS == 32, "block size");
  // block index of step t's first (or only) block
  static __device__ __forceinline__ int block(int t) {
    return BS == 16 ? t : BS == 32 ? (t >> 1) : 2 * t;
  }
};

// One work item of the decode kernel (unit = its id in the work order): a
// partition of one sequence for one KV head, all g query heads of that KV
// head.  smem holds MfmaLds<CDT, D>::kBytes bytes; item_lds passes the work
// item's sequence, its context length and the partition from the first wave
// to the others.
template <DT QDT, DT CDT, int D, int BS>
__device__ __forceinline__ void mfma_walk(const DecodePtrs& ptr, const DecodeParams& p, int unit,
                                          uint8_t* smem, float (*c_m)[16], float (*c_l)[16],
                                          int* item_lds) {
  using QS = typename Elem<QDT>::storage;
  using Raw = typename RawChunk<CDT>::type;
  using LDS = MfmaLds<CDT, D>;
  constexpr int E = Elem<CDT>::bytes;
  constexpr int NC = D / 16;                           // 16-row chunks per tile
  constexpr size_t kTileBytes = LDS::kTileBytes;       // one step's K (or V) image in LDS
  constexpr size_t kCacheTile = size_t(D) * BS * E;    // one (block, KV head) tile in a cache
  constexpr bool kStaged = CDT == DT::FP8;
  constexpr int kWaveLds = LDS::kWave;
  static_assert(!kStaged || kTileBytes % 1024 == 0, "a tile is copied 1 KiB per instruction");
  auto c_o = [&](int w, int hn, int d) -> float& {
    return reinterpret_cast<float*>(smem + w * kWaveLds)[hn * D + d];
  };

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int n = lane & 15;
  const int kq = lane >> 4;
  // Work items in id order, KV head fastest (dealt round-robin to the XCDs),
  // sequences in the longest-first order, as in the VALU kernel.
  const int kvh = unit % p.Hk;
  if (wid == 0) {                                      // one search per work-group
    int len = 0, pt = 0;
    const int s0 = longest_first_sequence(unit / p.Hk, p.np_run, p.bpp, ptr.context_lens, p.S,
                                          p.cap, pt, len);
    if (lane == 0) {
      item_lds[0] = s0;
      item_lds[1] = len;
      item_lds[2] = pt;
    }
  }
  __syncthreads();
  const int s = __builtin_amdgcn_readfirstlane(item_lds[0]);
  if (s < 0) return;                                   // past the last item: the group leaves
  const int l_raw = __builtin_amdgcn_readfirstlane(item_lds[1]);
  const int part = __builtin_amdgcn_readfirstlane(item_lds[2]);

  const int nb = tiles_of(l_raw, p.cap);               // 16-token steps
  const int L = tokens_of(l_raw, p.cap);
  const int nblk = (L + BS - 1) / BS;                  // blocks holding the tokens
  const int nparts = nb == 0 ? 1 : (nb + p.bpp - 1) / p.bpp;

  const int g = p.g;
  const int h = kvh * g + n;                            // this lane's query head (if n < g)
  const bool head_ok = n < g;
  // rows n >= g read head 0's q: their scores and sums are computed but
  // never written, and q is used as loaded, so that the first tiles are
  // requested without waiting for it
  typename Mfma<QDT>::vec qb[NC];
  {
    const QS* q = reinterpret_cast<const QS*>(ptr.query) + size_t(s) * p.q_stride +
                  size_t(head_ok ? h : 0) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      short4_t v = *reinterpret_cast<const short4_t*>(q + 16 * c + 4 * kq);
      qb[c] = Mfma<QDT>::from_bits(v);
    }
  }
  typename Mfma<QDT>::vec ident;
  {
    short4_t v;
    const short one = Mfma<QDT>::bits(1.0f);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (4 * kq + i == n) ? one : short(0);
    ident = Mfma<QDT>::from_bits(v);
  }

  // the sequence's steps are split into nparts nearly equal runs, and the
  // work-group's run among its waves the same way
  const int pj0 = (part * nb) / nparts;
  const int pj1 = ((part + 1) * nb) / nparts;
  const int j0 = pj0 + (wid * (pj1 - pj0)) / kWaves;
  const int j1 = pj0 + ((wid + 1) * (pj1 - pj0)) / kWaves;
  // At BLOCK_SIZE 32 the E4M3 walk takes whole blocks, and the 16-bit one
  // (head sizes up to 128) takes 32-token tiles at every block size (a
  // block, two or four).  The partition's and the waves' runs are then split in these
  // tiles (wb0 .. wb1 - 1).
  constexpr bool kWhole16 = !kStaged && NC <= 8;
  const int ntl32 = (nblk + 32 / BS - 1) / (32 / BS);
  const int pb0 = (part * ntl32) / nparts;
  const int pb1 = ((part + 1) * ntl32) / nparts;
  const int wb0 = pb0 + (wid * (pb1 - pb0)) / kWaves;
  const int wb1 = pb0 + ((wid + 1) * (pb1 - pb0)) / kWaves;
  const int32_t* bt = ptr.block_tables + size_t(s) * p.MB;
  // lane's 4 tokens of row n of each chunk, within its block's tile
  const int tok_in_block = BS == 8 ? 4 * (kq & 1) : 4 * kq;
  const size_t lane_off = size_t(kvh) * kCacheTile + (size_t(n) * BS + tok_in_block) * E;
  const size_t block_stride = size_t(p.Hk) * kCacheTile;
  constexpr size_t kChunkBytes = size_t(16) * BS * E;
  const uint8_t* kbase = ptr.kcache + lane_off;
  const uint8_t* vbase = ptr.vcache + lane_off;

  // online-softmax state of head n and the work on one step of 16 tokens
  // (tokens tb .. tb + 15): scores, softmax update, weighted sum.  okmask:
  // bit t says whether token tb + t comes from a valid block (at BLOCK_SIZE
  // 8 the step's two blocks are checked separately).  Kept as a lambda over
  // the kernel's locals: the same code as a member or free function compiled
  // to register spills in the FP8 variants.
  float m = -INFINITY, l = 0.f;
  float4_t o[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) o[c] = float4_t{0.f, 0.f, 0.f, 0.f};
  // kin: the K chunks as loaded (kT false: K[d][t], transposed here by an
  // MFMA against the identity; tokens that do not count are zeroed first
  // since the transpose mixes tokens) or already transposed by the LDS read
  // (kT true).
  auto block = [&](auto transposed, const short4_t (&kin)[NC], const Raw (&vraw)[NC], int tb,
                   uint32_t okmask) {
    constexpr bool kT = decltype(transposed)::value;
    const float4_t zero4 = {0.f, 0.f, 0.f, 0.f};
    short4_t kr[NC], vr[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      kr[c] = kin[c];
      vr[c] = to_operand<QDT, CDT>(vraw[c]);
    }
    auto counts = [&](int i) {                   // token tb + 4 kq + i
      return tb + 4 * kq + i < L && ((okmask >> (4 * kq + i)) & 1u);
    };
    if (tb + kTileTokens > L || okmask != 0xFFFFu) {   // tokens that may hold NaN
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (!counts(i)) {
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            if (!kT) kr[c][i] = 0;
            vr[c][i] = 0;
          }
        }
      }
    }

    // scores S^T[t][row], accumulated over the NC chunks of head_size
    float4_t st = zero4;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if constexpr (kT) {
        st = Mfma<QDT>::run(Mfma<QDT>::from_bits(kr[c]), qb[c], st);
      } else {
        const float4_t tt = Mfma<QDT>::run(Mfma<QDT>::from_bits(kr[c]), ident, zero4);  // K[4kq+i][n]
        short4_t tb16;
#pragma unroll
        for (int i = 0; i < 4; ++i) tb16[i] = Mfma<QDT>::bits(tt[i]);           // exact
        st = Mfma<QDT>::run(Mfma<QDT>::from_bits(tb16), qb[c], st);
      }
    }

    // online softmax for row n over tokens 4 kq + i
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = counts(i) ? st[i] * p.qk_scale : -INFINITY;
    float bm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    bm = fmaxf(bm, xor_lane<16>(bm));
    bm = fmaxf(bm, xor_lane<32>(bm));
    const float m_new = fmaxf(m, bm);
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_ref);
    m = m_new;

    short4_t ph, pl;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pr = fast_exp2(x[i] - m_ref);
      ph[i] = Mfma<QDT>::bits(pr);
      const float rest = pr - Mfma<QDT>::value(ph[i]);
      pl[i] = Mfma<QDT>::bits(rest);
      psum += Mfma<QDT>::value(ph[i]) + Mfma<QDT>::value(pl[i]);
    }
    l = fmaf(l, alpha, psum);

    // rescale the running sums only when some row's maximum moved (after the
    // first few blocks it rarely does); the test is wave-uniform
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
      for (int c = 0; c < NC; ++c) o[c] = o[c] * alpha;
    }
    // O^T[d][row] = sum_t V[d][t] P^T[t][row]
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float4_t acc = Mfma<QDT>::run(Mfma<QDT>::from_bits(vr[c]), Mfma<QDT>::from_bits(ph), o[c]);
      o[c] = Mfma<QDT>::run(Mfma<QDT>::from_bits(vr[c]), Mfma<QDT>::from_bits(pl), acc);
    }
  };
  auto valid = [&](int phys) { return static_cast<unsigned>(phys) < static_cast<unsigned>(p.NB); };
  // tokens of a step whose block(s) are valid
  auto step_mask = [&](int ia, int ib) -> uint32_t {
    if constexpr (BS == 8) return (valid(ia) ? 0x00FFu : 0u) | (valid(ib) ? 0xFF00u : 0u);
    else return valid(ia) ? 0xFFFFu : 0u;
  };

  // Decode with append: the wave whose steps include logical position L - 1
  // puts the new token into that step's tiles before reading its operands,
  // and stores them back.  The token is step t_new's token o_new.
  const bool appending = p.knew != nullptr && l_raw >= 1 && l_raw <= p.cap;
  const int t_new = appending ? (l_raw - 1) / kTileTokens : -1;
  const int o_new = (l_raw - 1) & (kTileTokens - 1);
  const size_t knew_row = (size_t(s) * p.kn_stride + size_t(kvh) * D) * Elem<QDT>::bytes;
  const size_t vnew_row = (size_t(s) * p.vn_stride + size_t(kvh) * D) * Elem<QDT>::bytes;

  // the lane's bytes of step t (block ids ia, ib) in a cache: at BLOCK_SIZE
  // 8 the lane's block is the step's first or second by its tokens, at 32
  // the step is the block's first or second half
  auto lane_at = [&](const uint8_t* base, int t, int ia, int ib) {
    const int id = BS == 8 && kq >= 2 ? ib : ia;
    const size_t half = BS == 32 ? size_t(t & 1) * kTileTokens * E : 0;
    return base + size_t(valid(id) ? id : 0) * block_stride + half;
  };
  auto load_k = [&](int t, int ia, int ib, Raw (&kr)[NC]) {
    const uint8_t* at = lane_at(kbase, t, ia, ib);
#pragma unroll
    for (int c = 0; c < NC; ++c) kr[c] = load_raw<CDT>(at + c * kChunkBytes);
  };
  auto load_v = [&](int t, int ia, int ib, Raw (&vr)[NC]) {
    const uint8_t* at = lane_at(vbase, t, ia, ib);
#pragma unroll
    for (int c = 0; c < NC; ++c) vr[c] = load_raw<CDT>(at + c * kChunkBytes);
  };

  if constexpr (!kStaged) {
    // append: before the walk, the wave patches the tiles of step t_new in
    // registers (lane (kq, n) holds tokens 4 kq .. 4 kq + 3 of row
    // 16 c + n) and stores them back to the addresses they are loaded from
    // (at BLOCK_SIZE 8 only the lanes of the block that holds the token);
    // the walk then reads them with the new token in place.
    const bool patch = kWhole16 ? (t_new >= 0 && t_new / 2 >= wb0 && t_new / 2 < wb1)
                                : (t_new >= j0 && t_new < j1);
    if (patch) {
      const int ia = bt[Steps<BS>::block(t_new)];
      const int ib = BS == 8 && 2 * t_new + 1 < nblk ? bt[2 * t_new + 1] : -1;
      const int id_new = BS == 8 && o_new >= 8 ? ib : ia;
      if (valid(id_new)) {
        Raw kr[NC], vr[NC];
        load_k(t_new, ia, ib, kr);
        load_v(t_new, ia, ib, vr);
        if (kq == o_new / 4) {
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            const int d = 16 * c + n;
            const short kb16 = short(new_token_bits<QDT, CDT>(p.knew + knew_row, d, 1.f));
            const short vb16 = short(new_token_bits<QDT, CDT>(p.vnew + vnew_row, d, 1.f));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              if (i == o_new % 4) {
                kr[c][i] = kb16;
                vr[c][i] = vb16;
              }
            }
          }
        }
        if (BS != 8 || (kq >= 2) == (o_new >= 8)) {
          uint8_t* kd = const_cast<uint8_t*>(lane_at(kbase, t_new, ia, ib));
          uint8_t* vd = const_cast<uint8_t*>(lane_at(vbase, t_new, ia, ib));
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            *reinterpret_cast<Raw*>(kd + c * kChunkBytes) = kr[c];
            *reinterpret_cast<Raw*>(vd + c * kChunkBytes) = vr[c];
          }
        }
        wait_vmem<0>();
      }
    }
  }

  if constexpr (kStaged && BS == 32) {
    // E4M3 at BLOCK_SIZE 32: the walk takes whole blocks (two 16-token
    // halves computed one after the other), and the partition's and the
    // waves' runs are split in blocks.  A block's K and V tiles are copied
    // whole (contiguous, 1 KiB per instruction, read once: nontemporal) into
    // two LDS images of the wave, [D][32] bytes each.  The next block's K
    // image is requested once the first half's operands and the second
    // half's K operands are in registers, its V image once the second half's
    // V operands are, so that it streams in while this block is computed.
    constexpr int kImg = D * 32;                        // bytes of one image
    constexpr int kQ = kImg / 1024;                      // copies per image
    static_assert(2 * kImg <= kWaveLds, "two whole-block images per wave");
    uint8_t* kimg = smem + wid * kWaveLds;
    uint8_t* vimg = kimg + kImg;
    const int b0 = wb0, b1 = wb1;
    const int b_new = appending ? (l_raw - 1) / 32 : -1;
    const int o_blk = (l_raw - 1) & 31;
    // this lane's 16 bytes of the first copy of block id's tile
    auto tile_at = [&](const uint8_t* cache, int id) {
      return cache + size_t(valid(id) ? id : 0) * block_stride + size_t(kvh) * kCacheTile +
             size_t(lane) * 16;
    };
    auto copy_img = [&](const uint8_t* cache, int id, uint8_t* img) {
      const uint8_t* g = tile_at(cache, id);
#pragma unroll
      for (int r = 0; r < kQ; ++r)
        __builtin_amdgcn_global_load_lds(g + r * 1024, (lds_void_t*)(img + r * 1024), 16, 0,
                                         kDmaNontemporal);
    };
    const uint32_t kt0 = lds_address(kimg) + kt_lane_offset32(kq, n);
    const uint32_t v0 = lds_address(vimg) + uint32_t(n * 32 + 4 * kq);
    for (int c0 = b0; c0 < b1; c0 += 64) {
      const int cnt = (b1 - c0) < 64 ? (b1 - c0) : 64;
      const int my_id = lane < cnt ? bt[c0 + lane] : 0;
      int id = __builtin_amdgcn_readlane(my_id, 0);
      copy_img(ptr.kcache, id, kimg);
      copy_img(ptr.vcache, id, vimg);
      for (int jj = 0; jj < cnt; ++jj) {
        const bool more = jj + 1 < cnt;
        const int nid = more ? __builtin_amdgcn_readlane(my_id, jj + 1) : 0;
        const int tb = (c0 + jj) * 32;
        wait_vmem<0>();                                  // this block's images have landed
        const bool ok = valid(id);
        if (ok && c0 + jj == b_new) {
          // the new token into both images (row d at d * 32 bytes), then
          // the images back to the block's tiles
          for (int d = lane; d < D; d += 64) {
            kimg[d * 32 + o_blk] = uint8_t(new_token_bits<QDT, CDT>(p.knew + knew_row, d, p.enc_k));
            vimg[d * 32 + o_blk] = uint8_t(new_token_bits<QDT, CDT>(p.vnew + vnew_row, d, p.enc_v));
          }
          uint8_t* kd = const_cast<uint8_t*>(tile_at(ptr.kcache, id));
          uint8_t* vd = const_cast<uint8_t*>(tile_at(ptr.vcache, id));
#pragma unroll
          for (int r = 0; r < kQ; ++r) {
            const int o = r * 1024 + lane * 16;
            *reinterpret_cast<u32x4_t*>(kd + r * 1024) = *reinterpret_cast<const u32x4_t*>(kimg + o);
            *reinterpret_cast<u32x4_t*>(vd + r * 1024) = *reinterpret_cast<const u32x4_t*>(vimg + o);
          }
          wait_vmem<0>();
        }
        const bool second = ok && tb + kTileTokens < L;   // the second half holds tokens
        u32x2_t ka[NC / 2], kb[NC / 2];
        Raw va[NC], vb[NC];
        if (ok) StagedKtV32<NC>::read(kt0, v0, ka, va);
        if (second) StagedKtV32<NC>::read_k(kt0 + kTileTokens, kb);
        if (more) copy_img(ptr.kcache, nid, kimg);
        if (ok) {
          short4_t kt[NC];
          kt_operands<QDT, CDT, NC>(ka, kt);
          block(std::true_type{}, kt, va, tb, 0xFFFFu);
        }
        if (second) StagedKtV32<NC>::read_v(v0 + kTileTokens, vb);
        if (more) copy_img(ptr.vcache, nid, vimg);
        if (second) {
          short4_t kt[NC];
          kt_operands<QDT, CDT, NC>(kb, kt);
          block(std::true_type{}, kt, vb, tb + kTileTokens, 0xFFFFu);
        }
        id = nid;
      }
    }
  } else if constexpr (kWhole16) {
    // 16-bit caches, 32-token tiles of NBT = 32 / BLOCK_SIZE consecutive
    // blocks, two 16-token halves each.  The tile's K is copied whole into an
    // LDS image of the wave (1 KiB per instruction, the blocks' tiles one
    // after the other) and read back transposed; its V is loaded to registers
    // whole, 16 bytes of a row per lane: lane (kq, n) holds tokens
    // 8 kq .. 8 kq + 7 of the tile in row 16 c + n (at BLOCK_SIZE 16 in block
    // kq / 2, at 8 all of block kq's), the first four for the first half and
    // the last four for the second.  A half's token slot 4 kq + i
    // is thus token 8 kq + 4 h + i of the tile, and the transposing read
    // points each lane at the same tokens: a relabelling inside the half
    // that the softmax and the weighted sums do not see.  Both halves'
    // scores come first (the next tile's K image is requested once they are
    // done), then one softmax update over the tile and both halves' products
    // with V (the next tile's V is requested after them).
    constexpr int NBT = 32 / BS;                        // blocks per tile
    constexpr int kImg = D * 64;                        // one tile's K
    constexpr int kBlkImg = D * BS * 2;                  // one block's K tile
    constexpr int kQB = (kBlkImg + 1023) / 1024;         // copies per block (the last partial)
    static_assert(kImg <= kWaveLds, "one K image per wave");
    static_assert(kBlkImg % 16 == 0, "a block tile is copied 16 bytes per lane");
    uint8_t* kimg = smem + wid * kWaveLds;
    const float4_t zero4 = {0.f, 0.f, 0.f, 0.f};
    auto tile_base = [&](const uint8_t* cache, int id) {
      return cache + size_t(valid(id) ? id : 0) * block_stride + size_t(kvh) * kCacheTile;
    };
    // the tile's blocks q = 0 .. NBT - 1 (block NBT t + q, id -1 past the
    // sequence's last block)
    auto copy_k = [&](const int (&ids)[NBT], int t) {
#pragma unroll
      for (int q = 0; q < NBT; ++q) {
        if (NBT * t + q >= nblk) continue;             // (uniform)
        const uint8_t* g = tile_base(ptr.kcache, ids[q]) + size_t(lane) * 16;
#pragma unroll
        for (int r = 0; r < kQB; ++r) {
          // a partial last copy: only the lanes inside the tile copy
          if (kBlkImg % 1024 == 0 || r * 1024 + lane * 16 < kBlkImg)
            __builtin_amdgcn_global_load_lds(g + r * 1024,
                                             (lds_void_t*)(kimg + q * kBlkImg + r * 1024), 16, 0,
                                             kDmaPrefix);
        }
      }
    };
    // this lane's V block (block kq * NBT / 4 of the tile) and its bytes
    auto lane_id = [&](const int (&ids)[NBT]) {
      if constexpr (NBT == 4) return kq == 0 ? ids[0] : kq == 1 ? ids[1] : kq == 2 ? ids[2] : ids[3];
      else if constexpr (NBT == 2) return kq < 2 ? ids[0] : ids[1];
      else return ids[0];
    };
    constexpr int kLanesPerRow = 4 / NBT;               // lanes (kq) sharing a block row
    const size_t v_lane = size_t(n) * (2 * BS) + size_t(kq % kLanesPerRow) * 16;
    constexpr int kVChunk = 16 * BS * 2;                 // bytes between chunks of a block tile
    auto load_vb = [&](int id, u32x4_t (&v)[NC]) {
      const uint8_t* g = tile_base(ptr.vcache, id) + v_lane;
#pragma unroll
      for (int c = 0; c < NC; ++c) v[c] = *reinterpret_cast<const u32x4_t*>(g + c * kVChunk);
    };
    auto read_k = [&](uint32_t a, u32x2_t (&k)[NC]) { StagedKt16T<NC, kVChunk>::read_k(a, k); };
    // the transposing read of lane (kq, n): row 4 kq + n / 4 of each chunk,
    // tokens 8 (n % 4) .. + 3 of the tile (in block (n % 4) * NBT / 4), + 4
    // tokens in the second half
    const int q4 = n & 3;
    const uint32_t kt0 = lds_address(kimg) +
                         uint32_t((q4 / kLanesPerRow) * kBlkImg + (4 * kq + (n >> 2)) * (2 * BS) +
                                  (q4 % kLanesPerRow) * 16);
    for (int c0 = wb0; c0 < wb1; c0 += 64) {
      const int cnt = (wb1 - c0) < 64 ? (wb1 - c0) : 64;
      int my_ids[NBT];
#pragma unroll
      for (int q = 0; q < NBT; ++q) {
        const int b = NBT * (c0 + lane) + q;
        my_ids[q] = lane < cnt && b < nblk ? bt[b] : -1;
      }
      int ids[NBT];
#pragma unroll
      for (int q = 0; q < NBT; ++q) ids[q] = __builtin_amdgcn_readlane(my_ids[q], 0);
      u32x4_t vb[NC];
      copy_k(ids, c0);
      asm volatile("" ::: "memory");                     // the K copies first
      load_vb(lane_id(ids), vb);
      for (int jj = 0; jj < cnt; ++jj) {
        const int t = c0 + jj;
        const bool more = jj + 1 < cnt;
        int nids[NBT];
#pragma unroll
        for (int q = 0; q < NBT; ++q) nids[q] = more ? __builtin_amdgcn_readlane(my_ids[q], jj + 1) : -1;
        const int tb = t * 32;
        wait_vmem<NC>();                                 // the K image has landed (V may not have)
        // blocks that count: any of the tile's (per lane: its own block)
        bool ok = false, all_ok = true;
#pragma unroll
        for (int q = 0; q < NBT; ++q) {
          ok = ok || valid(ids[q]);
          all_ok = all_ok && (NBT * t + q >= nblk || valid(ids[q]));
        }
        const bool lane_ok = valid(lane_id(ids));
        const bool second = ok && tb + 4 < L;            // the second half's first token is tb + 4
        float4_t st[2] = {zero4, zero4};
        if (ok) {
          u32x2_t kt[NC];
          read_k(kt0, kt);
#pragma unroll
          for (int c = 0; c < NC; ++c)
            st[0] = Mfma<QDT>::run(Mfma<QDT>::from_bits(__builtin_bit_cast(short4_t, kt[c])), qb[c], st[0]);
          if (second) {
            read_k(kt0 + 8, kt);
#pragma unroll
            for (int c = 0; c < NC; ++c)
              st[1] = Mfma<QDT>::run(Mfma<QDT>::from_bits(__builtin_bit_cast(short4_t, kt[c])), qb[c], st[1]);
          }
        }
        asm volatile("" ::: "memory");
        if (more) copy_k(nids, t + 1);
        if (ok) {
          // one softmax update over the tile's tokens that count
          auto tok = [&](int h, int i) { return tb + 8 * kq + 4 * h + i; };
          auto counts = [&](int h, int i) { return lane_ok && tok(h, i) < L; };
          float x[2][4];
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) x[h][i] = counts(h, i) ? st[h][i] * p.qk_scale : -INFINITY;
          float bm = -INFINITY;
#pragma unroll
          for (int h = 0; h < 2; ++h)
            bm = fmaxf(bm, fmaxf(fmaxf(x[h][0], x[h][1]), fmaxf(x[h][2], x[h][3])));
          bm = fmaxf(bm, xor_lane<16>(bm));
          bm = fmaxf(bm, xor_lane<32>(bm));
          const float m_new = fmaxf(m, bm);
          const float m_ref = m_new == -INFINITY ? 0.f : m_new;
          const float alpha = fast_exp2(m - m_ref);
          m = m_new;
          short4_t ph[2], pl[2];
          float psum = 0.f;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float pr = fast_exp2(x[h][i] - m_ref);
              ph[h][i] = Mfma<QDT>::bits(pr);
              const float rest = pr - Mfma<QDT>::value(ph[h][i]);
              pl[h][i] = Mfma<QDT>::bits(rest);
              psum += Mfma<QDT>::value(ph[h][i]) + Mfma<QDT>::value(pl[h][i]);
            }
          }
          l = fmaf(l, alpha, psum);
          if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
            for (int c = 0; c < NC; ++c) o[c] = o[c] * alpha;
          }
          // V of tokens that do not count (past L, or of a missing block)
          // may hold NaN: zeroed
          const bool partial = tb + 32 > L || !all_ok;
#pragma unroll
          for (int c = 0; c < NC; ++c) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              short4_t vv = __builtin_bit_cast(short4_t, h ? u32x2_t{vb[c].z, vb[c].w}
                                                           : u32x2_t{vb[c].x, vb[c].y});
              if (partial) {
#pragma unroll
                for (int i = 0; i < 4; ++i) vv[i] = counts(h, i) ? vv[i] : short(0);
              }
              float4_t acc = Mfma<QDT>::run(Mfma<QDT>::from_bits(vv), Mfma<QDT>::from_bits(ph[h]), o[c]);
              o[c] = Mfma<QDT>::run(Mfma<QDT>::from_bits(vv), Mfma<QDT>::from_bits(pl[h]), acc);
            }
          }
        }
        asm volatile("" ::: "memory");
        if (more) load_vb(lane_id(nids), vb);
#pragma unroll
        for (int q = 0; q < NBT; ++q) ids[q] = nids[q];
      }
#pragma unroll
      for (int q = 0; q < NBT; ++q) asm volatile("" ::"v"(my_ids[q]));
    }
  } else
  // Walk the wave's steps 64 at a time: ids fetched with one vector load
  // (two at BLOCK_SIZE 8) and read with readlane.  Loads are unconditional
  // (an id outside the pool reads block 0; its tokens are masked).
  for (int c0 = j0; c0 < j1; c0 += 64) {
    const int cnt = (j1 - c0) < 64 ? (j1 - c0) : 64;
    const int my_t = c0 + (lane < cnt ? lane : 0);
    const int my_ia = lane < cnt ? bt[Steps<BS>::block(my_t)] : 0;
    const int my_ib = BS == 8 && lane < cnt && 2 * my_t + 1 < nblk ? bt[2 * my_t + 1] : -1;
    auto ia_at = [&](int jj) { return __builtin_amdgcn_readlane(my_ia, jj); };
    auto ib_at = [&](int jj) { return BS == 8 ? __builtin_amdgcn_readlane(my_ib, jj) : -1; };
    if constexpr (kStaged) {
      // Step j+1's K and V images are copied into the other LDS stage while
      // step j is computed; each wave uses only its own kWaveLds bytes.
      constexpr int kPiece = 16;                        // bytes per lane per copy
      constexpr int kQ = int(kTileBytes) / (64 * kPiece); // copy instructions per image
      static_assert(BS != 32, "block size 32 walks whole blocks");
      constexpr int kPolicy = kDmaNontemporal;
      uint8_t* wbuf = smem + wid * kWaveLds;
      // global byte of image byte `o` (lane l of copy r: o = r * 64 kPiece +
      // l * kPiece) of step t in a cache, KV head kvh: the image is the tile
      // at 16, the two tiles at 8
      auto src = [&](const uint8_t* cache, int t, int ia, int ib, int o) {
        int id = ia;
        size_t in_tile;
        if constexpr (BS == 16) {
          in_tile = size_t(o);
        } else {
          id = o >= D * 8 ? ib : ia;
          in_tile = size_t(o >= D * 8 ? o - D * 8 : o);
        }
        return cache + size_t(valid(id) ? id : 0) * block_stride + size_t(kvh) * kCacheTile +
               in_tile;
      };
      auto issue = [&](int t, int ia, int ib, int stage) {
        uint8_t* sb = wbuf + stage * 2 * int(kTileBytes);
#pragma unroll
        for (int r = 0; r < kQ; ++r)
          __builtin_amdgcn_global_load_lds(src(ptr.kcache, t, ia, ib, (r * 64 + lane) * kPiece),
                                           (lds_void_t*)(sb + r * 64 * kPiece), kPiece, 0,
                                           kPolicy);
#pragma unroll
        for (int r = 0; r < kQ; ++r)
          __builtin_amdgcn_global_load_lds(src(ptr.vcache, t, ia, ib, (r * 64 + lane) * kPiece),
                                           (lds_void_t*)(sb + kTileBytes + r * 64 * kPiece),
                                           kPiece, 0, kPolicy);
      };
      // LDS addresses of this lane's K^T and V operand bytes in stage 0
      const uint32_t kt0 = lds_address(wbuf) + (BS == 8 ? kt_lane_offset8(kq, n, D)
                                                        : kt_lane_offset<CDT>(kq, n));
      const uint32_t v0 = lds_address(wbuf + kTileBytes) +
                          (BS == 8 ? v_lane_offset8(kq, n, D)
                                   : uint32_t((n * kTileTokens + 4 * kq) * E));
      issue(c0, ia_at(0), ib_at(0), 0);
      for (int jj = 0; jj < cnt; ++jj) {
        const int st = jj & 1;
        if (jj + 1 < cnt) {
          issue(c0 + jj + 1, ia_at(jj + 1), ib_at(jj + 1), st ^ 1);
          wait_vmem<2 * kQ>();                           // step jj's stage has landed
        } else {
          wait_vmem<0>();
        }
        const int ia = ia_at(jj), ib = ib_at(jj);
        const uint32_t ok = step_mask(ia, ib);
        if (ok != 0) {
          u32x2_t kraw[CDT == DT::FP8 ? NC / 2 : NC];
          Raw vr[NC];
          const uint32_t so = st * 2 * uint32_t(kTileBytes);
          if (c0 + jj == t_new) {
            // the new token into the staged images (row d at d * 16 bytes),
            // then the images back to the caches: the bytes of the block
            // that holds the token, with the mapping they were copied with
            uint8_t* sb = wbuf + so;
            // the token's byte of image row d
            const int at_new = BS == 8 ? (o_new >= 8 ? D * 8 + o_new - 8 : o_new) : o_new;
            const int row_bytes = BS == 8 ? 8 : kTileTokens;
            for (int d = lane; d < D; d += 64) {
              sb[d * row_bytes + at_new] =
                  uint8_t(new_token_bits<QDT, CDT>(p.knew + knew_row, d, p.enc_k));
              sb[kTileBytes + d * row_bytes + at_new] =
                  uint8_t(new_token_bits<QDT, CDT>(p.vnew + vnew_row, d, p.enc_v));
            }
            const int id_new = BS == 8 && o_new >= 8 ? ib : ia;
            if (valid(id_new)) {
#pragma unroll
              for (int r = 0; r < kQ; ++r) {
                const int o = (r * 64 + lane) * kPiece;
                if (BS == 8 && (o >= D * 8) != (o_new >= 8)) continue;   // the other block
                uint8_t* kd = const_cast<uint8_t*>(src(ptr.kcache, c0 + jj, ia, ib, o));
                uint8_t* vd = const_cast<uint8_t*>(src(ptr.vcache, c0 + jj, ia, ib, o));
                if constexpr (kPiece == 16) {
                  *reinterpret_cast<u32x4_t*>(kd) = *reinterpret_cast<const u32x4_t*>(sb + o);
                  *reinterpret_cast<u32x4_t*>(vd) =
                      *reinterpret_cast<const u32x4_t*>(sb + kTileBytes + o);
                } else {
                  *reinterpret_cast<uint32_t*>(kd) = *reinterpret_cast<const uint32_t*>(sb + o);
                  *reinterpret_cast<uint32_t*>(vd) =
                      *reinterpret_cast<const uint32_t*>(sb + kTileBytes + o);
                }
              }
            }
            wait_vmem<0>();                              // counts stay exact for the copies
          }
          if constexpr (BS == 8) StagedKtV8<NC>::read(kt0 + so, v0 + so, kraw, vr);
          else StagedKtV<CDT, NC>::read(kt0 + so, v0 + so, kraw, vr);
          short4_t kt[NC];
          kt_operands<QDT, CDT, NC>(kraw, kt);
          block(std::true_type{}, kt, vr, (c0 + jj) * kTileTokens, ok);
        }
      }
    } else {
      auto as_operands = [&](const Raw (&kraw)[NC]) {
        struct Ops { short4_t v[NC]; } r;
#pragma unroll
        for (int c = 0; c < NC; ++c) r.v[c] = to_operand<QDT, CDT>(kraw[c]);
        return r;
      };
      // K tiles are double-buffered in registers (step j+1's K is in flight
      // while step j is computed) and step j's V is issued just before step
      // j+1's K, so that the weighted sum waits for V(j) only.
      Raw ka[NC], kb[NC], vc[NC];
      int ia = ia_at(0), iab = ib_at(0);
      load_k(c0, ia, iab, ka);
      int jj = 0;
      for (; jj + 1 < cnt; jj += 2) {
        const int ib = ia_at(jj + 1), ibb = ib_at(jj + 1);
        load_v(c0 + jj, ia, iab, vc);
        load_k(c0 + jj + 1, ib, ibb, kb);
        if (const uint32_t ok = step_mask(ia, iab))
          block(std::false_type{}, as_operands(ka).v, vc, (c0 + jj) * kTileTokens, ok);
        const int nx = jj + 2 < cnt ? jj + 2 : jj + 1;
        const int ia2 = ia_at(nx), iab2 = ib_at(nx);
        load_v(c0 + jj + 1, ib, ibb, vc);
        load_k(c0 + nx, ia2, iab2, ka);
        if (const uint32_t ok = step_mask(ib, ibb))
          block(std::false_type{}, as_operands(kb).v, vc, (c0 + jj + 1) * kTileTokens, ok);
        ia = ia2;
        iab = iab2;
      }
      if (jj < cnt) {
        load_v(c0 + jj, ia, iab, vc);
        if (const uint32_t ok = step_mask(ia, iab))
          block(std::false_type{}, as_operands(ka).v, vc, (c0 + jj) * kTileTokens, ok);
      }
    }
  }
  l += xor_lane<16>(l);
  l += xor_lane<32>(l);

  // combine the waves of the work-group through LDS
  if (head_ok) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int i = 0; i < 4; ++i) c_o(wid, n, 16 * c + 4 * kq + i) = o[c][i];
    }
    if (kq == 0) {
      c_m[wid][n] = m;
      c_l[wid][n] = l;
    }
  }
  __syncthreads();
  const bool direct = nparts == 1;
  for (int idx = threadIdx.x; idx < g * D; idx += 64 * kWaves) {
    const int hn = idx / D, d = idx % D;
    float Mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) Mx = fmaxf(Mx, c_m[k][hn]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) {
      const float wk = c_m[k][hn] == -INFINITY ? 0.f : fast_exp2(c_m[k][hn] - Mx);
      num = fmaf(wk, c_o(k, hn, d), num);
      den = fmaf(wk, c_l[k][hn], den);
    }
    const int hq = kvh * g + hn;
    if (direct) {
      QS* out = reinterpret_cast<QS*>(ptr.out) + size_t(s) * p.o_stride + size_t(hq) * D;
      out[d] = from_f32<QDT>(den > 0.f ? num * (p.v_scale / den) : 0.f);
    } else {
      const size_t base = (size_t(s) * p.H + hq) * p.np + part;
      if (d == 0) {
        p.ws_m[base] = Mx;
        p.ws_l[base] = den;
      }
      p.ws_acc[base * D + d] = num;
    }
  }
}

template <DT QDT, DT CDT, int D, int BS>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(4)))
void decode_mfma_kernel(DecodePtrs ptr, DecodeParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[MfmaLds<CDT, D>::kBytes];
  __shared__ float c_m[kWaves][16], c_l[kWaves][16];
  __shared__ int item[3];
  mfma_walk<QDT, CDT, D, BS>(ptr, p, blockIdx.x, smem, c_m, c_l, item);
}

// Head sizes 192 and 256 (16-bit caches): 12 or 16 chunks of 16 rows per
// tile need about 200 registers per lane for the query, the accumulators and
// the double-buffered tiles, so these run at 2 waves per SIMD.
template <DT QDT, DT CDT, int D, int BS>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2)))
void decode_mfma_wide_kernel(DecodePtrs ptr, DecodeParams p) {
  static_assert(CDT != DT::FP8 && D > 128, "wide head sizes, 16-bit caches");
  __shared__ __attribute__((aligned(16))) uint8_t smem[MfmaLds<CDT, D>::kBytes];
  __shared__ float c_m[kWaves][16], c_l[kWaves][16];
  __shared__ int item[3];
  mfma_walk<QDT, CDT, D, BS>(ptr, p, blockIdx.x, smem, c_m, c_l, item);
}

// Prefix pass of a shared-prefix batch.  The sequences of a group share their
// first P blocks (parallel samples of one prompt, [L3] "共享前缀"; [TGI] §4:
// prefix reuse).  A work-group takes one run of at most ppb (16) of those blocks
// for one KV head and up to 4 x 16 of the group's query rows (row = member *
// g + head offset); each K/V tile of the run is copied into LDS once and read
// by all four waves, one 16-row tile each, so the prefix is read from memory
// once per group instead of once per member.  Each row's (max, sum, weighted
// sum) goes to workspace slot `run`; runs past the prefix write empty
// partials, so that the merge can take every slot.
template <DT CDT, int D>
struct PrefixLds {                                        // two pairs of K/V stages, shared
  static constexpr int kTile = D * kBlockSize * Elem<CDT>::bytes;
  static constexpr int kStages = 4;
  static constexpr int kBytes = kStages * 2 * kTile;
};

template <DT QDT, DT CDT, int D>
__device__ __forceinline__ void prefix_walk(const DecodePtrs& ptr, const DecodeParams& p,
                                            int unit, uint8_t* smem) {
  using QS = typename Elem<QDT>::storage;
  using Raw = typename RawChunk<CDT>::type;
  constexpr int E = Elem<CDT>::bytes;
  constexpr int NC = D / 16;
  constexpr int kTile = PrefixLds<CDT, D>::kTile;
  constexpr int kQ = kTile / 1024;                      // copy instructions per tile
  constexpr int kMine = (2 * kQ + kWaves - 1) / kWaves; // copy instructions per wave and stage
  static_assert(kTile % 1024 == 0, "a tile is copied 1 KiB per instruction");

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int n = lane & 15;
  const int kq = lane >> 4;
  int t = unit;
  const int kvh = t % p.Hk;
  t /= p.Hk;
  const int run = t % p.npp;
  t /= p.npp;
  const int grp = t % p.G;
  const int round = t / p.G;

  int gs = p.group_starts[grp], ge = p.group_starts[grp + 1];
  gs = gs < 0 ? 0 : (gs > p.S ? p.S : gs);
  ge = ge < gs ? gs : (ge > p.S ? p.S : ge);
  const int rows = (ge - gs) * p.g;
  if (round * kWaves * 16 >= rows) return;               // no rows for this work-group
  int P = p.group_prefix[grp];
  P = P < 0 ? 0 : (P > p.MB ? p.MB : P);
  const int b0 = run * p.ppb;
  const int b1 = b0 + p.ppb < P ? b0 + p.ppb : P;

  const int row = (round * kWaves + wid) * 16 + n;
  const bool row_ok = row < rows;
  const int seq = gs + (row_ok ? row / p.g : 0);
  const int head = kvh * p.g + (row_ok ? row % p.g : 0);
  // rows past the group read its first row's q (results never written)
  typename Mfma<QDT>::vec qb[NC];
  {
    const QS* q = reinterpret_cast<const QS*>(ptr.query) + size_t(seq) * p.q_stride +
                  size_t(head) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      short4_t v = *reinterpret_cast<const short4_t*>(q + 16 * c + 4 * kq);
      qb[c] = Mfma<QDT>::from_bits(v);
    }
  }
  const int L = P * kBlockSize;                         // prefix blocks are full
  float m = -INFINITY, l = 0.f;
  float4_t o[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) o[c] = float4_t{0.f, 0.f, 0.f, 0.f};
  // LDS addresses of this lane's K^T and V operands in stage 0
  const uint32_t kt0 = lds_address(smem) + kt_lane_offset<CDT>(kq, n);
  const uint32_t v0 = lds_address(smem + kTile + (n * kBlockSize + 4 * kq) * E);
  // Two blocks (tokens tb .. tb + 31) per step: scores of both, one
  // online-softmax update over the 32 tokens, then both weighted sums.
  // use_a / use_b (wave-uniform) say whether each block is read at all (a
  // block outside the pool, or past the run, contributes nothing).
  auto block2 = [&](uint32_t so_a, uint32_t so_b, bool use_a, bool use_b, int tb) {
    const float4_t zero4 = {0.f, 0.f, 0.f, 0.f};
    auto scores = [&](uint32_t so, Raw (&vraw)[NC]) {
      u32x2_t kraw[CDT == DT::FP8 ? NC / 2 : NC];
      StagedKtV<CDT, NC>::read(kt0 + so, v0 + so, kraw, vraw);
      short4_t kt[NC];
      kt_operands<QDT, CDT, NC>(kraw, kt);
      float4_t st = zero4;
#pragma unroll
      for (int c = 0; c < NC; ++c) st = Mfma<QDT>::run(Mfma<QDT>::from_bits(kt[c]), qb[c], st);
      return st;
    };
    Raw va[NC], vb[NC];
    float x[8];
    {
      const float4_t sa = use_a ? scores(so_a, va) : zero4;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        x[i] = (use_a && tb + 4 * kq + i < L) ? sa[i] * p.qk_scale : -INFINITY;
    }
    {
      const float4_t sb = use_b ? scores(so_b, vb) : zero4;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        x[4 + i] = (use_b && tb + 16 + 4 * kq + i < L) ? sb[i] * p.qk_scale : -INFINITY;
    }

    // online softmax for row n over tokens 4 kq + i of both blocks
    float bm = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) bm = fmaxf(bm, x[i]);
    bm = fmaxf(bm, xor_lane<16>(bm));
    bm = fmaxf(bm, xor_lane<32>(bm));
    const float m_new = fmaxf(m, bm);
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_ref);
    m = m_new;

    short4_t ph[2], pl[2];
    float psum = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pr = fast_exp2(x[4 * h + i] - m_ref);
        ph[h][i] = Mfma<QDT>::bits(pr);
        const float rest = pr - Mfma<QDT>::value(ph[h][i]);
        pl[h][i] = Mfma<QDT>::bits(rest);
        psum += Mfma<QDT>::value(ph[h][i]) + Mfma<QDT>::value(pl[h][i]);
      }
    }
    l = fmaf(l, alpha, psum);

    // rescale the running sums only when some row's maximum moved (after the
    // first few blocks it rarely does); the test is wave-uniform
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
      for (int c = 0; c < NC; ++c) o[c] = o[c] * alpha;
    }
    // O^T[d][row] = sum_t V[d][t] P^T[t][row], block by block
    auto weighted = [&](const Raw (&vraw)[NC], short4_t phh, short4_t pll) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const short4_t vr = to_operand<QDT, CDT>(vraw[c]);
        float4_t acc = Mfma<QDT>::run(Mfma<QDT>::from_bits(vr), Mfma<QDT>::from_bits(phh), o[c]);
        o[c] = Mfma<QDT>::run(Mfma<QDT>::from_bits(vr), Mfma<QDT>::from_bits(pll), acc);
      }
    };
    if (use_a) weighted(va, ph[0], pl[0]);
    if (use_b) weighted(vb, ph[1], pl[1]);
  };

  if (b0 < b1) {
    const int cnt = b1 - b0;                            // <= 64
    const int32_t* bt = ptr.block_tables + size_t(gs) * p.MB + b0;
    const int my_id = lane < cnt ? bt[lane] : 0;
    auto id_at = [&](int jj) { return __builtin_amdgcn_readlane(my_id, jj); };
    auto valid = [&](int phys) {
      return static_cast<unsigned>(phys) < static_cast<unsigned>(p.NB);
    };
    const size_t block_stride = size_t(p.Hk) * kTile;
    const uint32_t lane_bytes = uint32_t(lane) * 16;
    // this wave's share of the 2 kQ copy instructions of a stage: i = wid,
    // wid + 4, ...; the tile address is wave-uniform, only lane * 16 varies
    auto issue = [&](int phys, int stage) {
      const size_t tile = size_t(valid(phys) ? phys : 0) * block_stride + size_t(kvh) * kTile;
#pragma unroll
      for (int k = 0; k < kMine; ++k) {
        const int i = wid + k * kWaves;
        if (i < 2 * kQ) {
          const uint8_t* src = (i < kQ ? ptr.kcache : ptr.vcache) + tile + (i % kQ) * 1024;
          __builtin_amdgcn_global_load_lds(src + lane_bytes,
                                           (lds_void_t*)(smem + stage * 2 * kTile + i * 1024),
                                           16, 0, kDmaPrefix);
        }
      }
    };
    // Pairs of blocks: pair q's two blocks go to stages 2 (q % 2) and
    // 2 (q % 2) + 1.  Pairs 0 and 1 are requested up front; after the barrier
    // of pair q every wave is done with pair q - 1, whose stages then take
    // pair q + 1, which loads while pair q is computed.
    const int npairs = (cnt + 1) / 2;
    auto issue_pair = [&](int q) {
      issue(id_at(2 * q), 2 * (q & 1));
      if (2 * q + 1 < cnt) issue(id_at(2 * q + 1), 2 * (q & 1) + 1);
    };
    issue_pair(0);
    if (npairs > 1) issue_pair(1);
    for (int q = 0; q < npairs; ++q) {
      if (q == 0 && npairs > 1) {                       // pair 1 may still be in flight
        if (2 + 1 < cnt) wait_vmem<2 * kMine>();
        else wait_vmem<kMine>();
      } else {
        wait_vmem<0>();
      }
      // every wave's copies of pair q landed, and every wave is done with
      // pair q - 1, whose stages are refilled next
      __builtin_amdgcn_s_barrier();
      if (q >= 1 && q + 1 < npairs) issue_pair(q + 1);
      const int ja = 2 * q, jb = 2 * q + 1;
      const bool use_a = valid(id_at(ja));
      const bool use_b = jb < cnt && valid(id_at(jb < cnt ? jb : ja));
      const uint32_t so = (q & 1) * 4 * uint32_t(kTile);
      block2(so, so + 2 * uint32_t(kTile), use_a, use_b, (b0 + ja) * kBlockSize);
    }
  }
  l += xor_lane<16>(l);
  l += xor_lane<32>(l);

  if (row_ok) {
    const size_t base = (size_t(seq) * p.H + head) * p.np + run;
    if (b0 < b1) {                                      // an empty run leaves l = 0 only
#pragma unroll
      for (int c = 0; c < NC; ++c)
        *reinterpret_cast<float4_t*>(p.ws_acc + base * D + 16 * c + 4 * kq) = o[c];
    }
    if (kq == 0) {
      p.ws_m[base] = m;
      p.ws_l[base] = l;
    }
  }
}

template <DT QDT, DT CDT, int D>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(3)))
void decode_prefix_kernel(DecodePtrs ptr, DecodeParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[PrefixLds<CDT, D>::kBytes];
  prefix_walk<QDT, CDT, D>(ptr, p, blockIdx.x, smem);
}

// Shared-prefix batches on the matrix cores with no partial results.  The
// sequences of a group share their first P blocks (parallel samples of one
// prompt, [L3] "共享前缀"; [TGI] §4: prefix reuse).  A work-group takes one
// 16-row tile of the group's query rows for one KV head: gm = 16 / g members
// x their g query heads (row n = member n / g, head n % g).  Its walk list is
// the P prefix blocks (every row attends) followed by each member's own
// blocks P .. nb - 1 (only that member's rows attend; the others' scores are
// -inf, which leaves their state unchanged); element k goes to wave k mod NW.
// The waves combine through LDS and write the final output: there is no
// workspace and no merge.  Each prefix tile is read by the group's
// ceil(members / gm) tiles; their work-groups get ids that are equal mod 8, so
// they run on one XCD, and the interleaved split has all of them sweep the
// prefix front to back at about the same pace, so that all but the first
// find its blocks in that XCD's L2 (with contiguous per-wave runs, whose
// bounds depend on each tile's suffix lengths, the tiles read the prefix at
// different times and fetched it about twice from memory).
template <DT QDT, DT CDT, int D, int NW>
__device__ __forceinline__ void group_walk(const DecodePtrs& ptr, const DecodeParams& p, int id,
                                           uint8_t* smem, float (*c_m)[16], float (*c_l)[16]) {
  using QS = typename Elem<QDT>::storage;
  using Raw = typename RawChunk<CDT>::type;
  using LDS = MfmaLds<CDT, D>;
  constexpr int E = Elem<CDT>::bytes;
  constexpr int NC = D / 16;
  constexpr size_t kTileBytes = LDS::kTileBytes;
  constexpr bool kStaged = CDT == DT::FP8;
  constexpr int kWaveLds = LDS::kWave;
  static_assert(!kStaged || kTileBytes % 1024 == 0, "a tile is copied 1 KiB per instruction");
  auto c_o = [&](int w, int hn, int d) -> float& {
    return reinterpret_cast<float*>(smem + w * kWaveLds)[hn * D + d];
  };

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int n = lane & 15;
  const int kq = lane >> 4;
  // id -> (group, KV head) pair and tile: pair = 8 (id / 8 / gt) + id % 8,
  // tile = (id / 8) % gt, so a pair's tiles are ids equal mod 8
  const int pair = (id / 8 / p.gt) * 8 + id % 8;
  const int tile = (id / 8) % p.gt;
  if (pair >= p.G * p.Hk) return;
  const int grp = pair / p.Hk;
  const int kvh = pair % p.Hk;
  int gs = __builtin_amdgcn_readfirstlane(p.group_starts[grp]);
  int ge = __builtin_amdgcn_readfirstlane(p.group_starts[grp + 1]);
  gs = gs < 0 ? 0 : (gs > p.S ? p.S : gs);
  ge = ge < gs ? gs : (ge > p.S ? p.S : ge);
  const int s0 = gs + tile * p.gm;                      // the tile's first member
  if (s0 >= ge) return;                                 // the group has fewer tiles
  const int nm = ge - s0 < p.gm ? ge - s0 : p.gm;       // members in the tile
  const int g = p.g;
  const int rows = nm * g;
  const bool row_ok = n < rows;
  const int member = row_ok ? n / g : 0;                // this lane's row: member, head
  const int h = kvh * g + (row_ok ? n % g : 0);
  int P = __builtin_amdgcn_readfirstlane(p.group_prefix[grp]);
  P = P < 0 ? 0 : (P > p.MB ? p.MB : P);
  // per member j (at most 8: g >= 2), with wave-uniform indices only: where
  // its blocks start in the walk list, its token count, and the block that
  // receives its new token (append: the block holding position L - 1 when
  // 1 <= L <= cap and that block lies past the shared prefix; the token
  // count then is the raw length), packed as 2 L + (1 if it has one).  The
  // lengths come through the scalar cache: vector loads issued now would
  // queue behind the tile loads of the waves already walking.
  constexpr int kMaxMembers = 8;
  int m_start[kMaxMembers], m_Ln[kMaxMembers];
  int total = P;                                        // length of the walk list
  // (all eight requested before any is used -- the asm keeps the compiler
  // from sinking each load into the branch that uses it -- with indices
  // clamped into the array; so are the block ids of the wave's first two
  // elements of the list when they are prefix blocks, which need no lengths)
  int lens[kMaxMembers];
#pragma unroll
  for (int j = 0; j < kMaxMembers; ++j) lens[j] = scalar_ptr(ptr.context_lens)[s0 + j < ge ? s0 + j : ge - 1];
  const int* prow = ptr.block_tables + size_t(s0) * p.MB;
  const int pid0 = scalar_ptr(prow)[wid < P ? wid : 0];
  const int pid1 = scalar_ptr(prow)[wid + NW < P ? wid + NW : 0];
  asm volatile("" ::"s"(lens[0]), "s"(lens[1]), "s"(lens[2]), "s"(lens[3]), "s"(lens[4]),
               "s"(lens[5]), "s"(lens[6]), "s"(lens[7]), "s"(pid0), "s"(pid1));
#pragma unroll
  for (int j = 0; j < kMaxMembers; ++j) {
    const int l_raw = j < nm ? lens[j] : 0;
    const int nb = tiles_of(l_raw, p.cap);
    m_start[j] = total;
    const bool has_new = j < nm && p.knew != nullptr && l_raw >= 1 && l_raw <= p.cap &&
                         (l_raw - 1) / kBlockSize >= P;
    m_Ln[j] = 2 * tokens_of(l_raw, p.cap) + (has_new ? 1 : 0);
    total += j < nm && nb > P ? nb - P : 0;
  }
  auto new_block = [](int Ln) { return (Ln & 1) ? ((Ln >> 1) - 1) / kBlockSize : -1; };
  // walk-list element k (wave-uniform) -> its member (-1: a prefix block)
  // and its block index in that member's table row
  auto list_entry = [&](int k, int& mem, int& j) {
    mem = -1;
    j = k;
    if (k >= P) {
      int mm = 0, start = m_start[0];
#pragma unroll
      for (int jm = 1; jm < kMaxMembers; ++jm) {
        if (jm < nm && k >= m_start[jm]) {
          mm = jm;
          start = m_start[jm];
        }
      }
      mem = mm;
      j = P + (k - start);
    }
  };
  auto valid = [&](int phys) { return static_cast<unsigned>(phys) < static_cast<unsigned>(p.NB); };
  // The wave's elements of the walk list are k = wid, wid + NW, wid + 2 NW,
  // ... (interleaved, so that the tiles of a group sweep the prefix front to
  // back at the same pace and find its blocks in L2).  The first two block
  // ids come through the scalar cache: the walk starts from them without
  // waiting for the vector load of the rest.
  const int n_el = total > wid ? (total - wid + NW - 1) / NW : 0;
  auto scalar_block = [&](int k) {
    int mem, j;
    list_entry(k, mem, j);
    return scalar_ptr(ptr.block_tables)[size_t(s0 + (mem < 0 ? 0 : mem)) * p.MB + j];
  };
  const int id0 = wid < P ? pid0 : n_el > 0 ? scalar_block(wid) : -1;
  const int id1 = wid + NW < P ? pid1 : n_el > 1 ? scalar_block(wid + NW) : id0;

  // rows n >= rows read row 0's q: their results are never written
  typename Mfma<QDT>::vec qb[NC];
  auto load_q = [&]() {
    const QS* q = reinterpret_cast<const QS*>(ptr.query) + size_t(s0 + member) * p.q_stride +
                  size_t(h) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      short4_t v = *reinterpret_cast<const short4_t*>(q + 16 * c + 4 * kq);
      qb[c] = Mfma<QDT>::from_bits(v);
    }
  };
  const size_t lane_off = size_t(kvh) * kTileBytes + (size_t(n) * kBlockSize + 4 * kq) * E;
  const size_t block_stride = size_t(p.Hk) * kTileBytes;
  constexpr size_t kChunkBytes = size_t(16) * kBlockSize * E;
  const uint8_t* vbase = ptr.vcache + lane_off;
  // the new token of the sequence s0 + mem: byte offsets of its key and
  // value rows for this KV head
  auto new_rows = [&](int mem) {
    const size_t sq = size_t(s0 + mem);
    return std::pair<size_t, size_t>((sq * p.kn_stride + size_t(kvh) * D) * Elem<QDT>::bytes,
                                     (sq * p.vn_stride + size_t(kvh) * D) * Elem<QDT>::bytes);
  };

  // 16-bit caches, append: the new tokens whose blocks are elements of this
  // wave's walk go straight into their tiles before the walk (row d at
  // 16 d + offset elements), with nothing waited for.  Before the walk loads
  // such a tile it waits for all of its own memory operations, these stores
  // among them, so it reads the tile with the token in place (by then the
  // wait is mostly for the previous tile's loads, which its block needs
  // anyway); once the tile has arrived it stores the whole tile back from
  // registers, so that every line of the tile is written in full.  The tile
  // is its member's own block, read by this wave alone.  (Loading, patching
  // and storing each such tile before the walk, with a wait for the stores,
  // kept the patching waves 5-20 us behind the others of their work-group.)
  // E4M3 caches patch the staged tile inside the walk instead.
  auto store_new_tokens = [&]() {
    if constexpr (!kStaged) {
      static_assert(E == 2, "16-bit caches");          // bit patterns, stored as such
      constexpr int kR = (D + 63) / 64;
#pragma unroll
      for (int jm = 0; jm < kMaxMembers; ++jm) {
        const int nbk = new_block(m_Ln[jm]);
        if (nbk >= 0 && (m_start[jm] + nbk - P) % NW == wid) {
          const int bid = scalar_ptr(ptr.block_tables)[size_t(s0 + jm) * p.MB + nbk];
          if (valid(bid)) {
            const int o_new = ((m_Ln[jm] >> 1) - 1) & (kBlockSize - 1);
            const auto nr = new_rows(jm);
            uint16_t kv[kR], vv[kR];
#pragma unroll
            for (int r = 0; r < kR; ++r) {
              const int d = lane + 64 * r < D ? lane + 64 * r : D - 1;
              kv[r] = uint16_t(new_token_bits<QDT, CDT>(p.knew + nr.first, d, 1.f));
              vv[r] = uint16_t(new_token_bits<QDT, CDT>(p.vnew + nr.second, d, 1.f));
            }
            const size_t toff = size_t(bid) * block_stride + size_t(kvh) * kTileBytes;
            uint16_t* kt = reinterpret_cast<uint16_t*>(const_cast<uint8_t*>(ptr.kcache) + toff);
            uint16_t* vt = reinterpret_cast<uint16_t*>(const_cast<uint8_t*>(ptr.vcache) + toff);
#pragma unroll
            for (int r = 0; r < kR; ++r) {
              const int d = lane + 64 * r;
              if (d < D) {
                kt[d * kBlockSize + o_new] = kv[r];
                vt[d * kBlockSize + o_new] = vv[r];
              }
            }
          }
        }
      }
    }
  };
  store_new_tokens();                 // (called inside the walk it made the walk spill)

  // row n's online-softmax state and the work on one block of 16 tokens
  // (tokens tb .. tb + 15 of a sequence of L tokens): the arithmetic of
  // mfma_walk's block(), with `act` (per row) masking rows that do not
  // attend to this block
  float m = -INFINITY, l = 0.f;
  float4_t o[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) o[c] = float4_t{0.f, 0.f, 0.f, 0.f};
  // the scores st (S^T of the block, from the K^T operands and q) are
  // computed by the caller; then the online softmax and the weighted sum
  auto finish = [&](float4_t st, const Raw (&vraw)[NC], int tb, int L, bool act) {
    short4_t vr[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) vr[c] = to_operand<QDT, CDT>(vraw[c]);
    if (tb + kBlockSize > L) {          // zero tail tokens: they may hold NaN
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (tb + 4 * kq + i >= L) {
#pragma unroll
          for (int c = 0; c < NC; ++c) vr[c][i] = 0;
        }
      }
    }
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      x[i] = (act && tb + 4 * kq + i < L) ? st[i] * p.qk_scale : -INFINITY;
    float bm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    bm = fmaxf(bm, xor_lane<16>(bm));
    bm = fmaxf(bm, xor_lane<32>(bm));
    const float m_new = fmaxf(m, bm);
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_ref);
    m = m_new;
    short4_t ph, pl;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pr = fast_exp2(x[i] - m_ref);
      ph[i] = Mfma<QDT>::bits(pr);
      const float rest = pr - Mfma<QDT>::value(ph[i]);
      pl[i] = Mfma<QDT>::bits(rest);
      psum += Mfma<QDT>::value(ph[i]) + Mfma<QDT>::value(pl[i]);
    }
    l = fmaf(l, alpha, psum);
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
      for (int c = 0; c < NC; ++c) o[c] = o[c] * alpha;
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float4_t acc = Mfma<QDT>::run(Mfma<QDT>::from_bits(vr[c]), Mfma<QDT>::from_bits(ph), o[c]);
      o[c] = Mfma<QDT>::run(Mfma<QDT>::from_bits(vr[c]), Mfma<QDT>::from_bits(pl), acc);
    }
  };
  // K^T operands read from a stage (no tail zeroing: a token's NaN stays in
  // its own score, which is masked)
  auto block = [&](const short4_t (&kt)[NC], const Raw (&vraw)[NC], int tb, int L, bool act) {
    float4_t st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) st = Mfma<QDT>::run(Mfma<QDT>::from_bits(kt[c]), qb[c], st);
    finish(st, vraw, tb, L, act);
  };

  // Elements c0 .. c0 + cnt - 1 of the wave's list (1 <= cnt <= 64; first:
  // the first chunk, which starts from id0 / id1 and loads q behind its first
  // tile).  Lane i describes element c0 + i: its block id, its block index j
  // in the table and, packed as 16 L + member + 1, the token count L of its
  // sequence and its member (-1: a prefix block, every row attends; L < 2^26,
  // the host bounds the table), and whether the sequence's new token goes
  // into it (append).  Lanes past cnt describe the chunk's last element, so
  // that the table load needs no branch.
  auto walk_chunk = [&](int c0, int cnt, bool first) {
    int e_id, e_j, e_Lm;
    bool e_new;
    {
      const int k = wid + (c0 + (lane < cnt ? lane : cnt - 1)) * NW;   // list index
      int e_L, e_mem = -1, j;
      if (k < P) {
        j = k;
        e_L = P * kBlockSize;                           // prefix blocks are full
        e_new = false;
      } else {
        // the member whose part of the list holds element k: the last one
        // that starts at or before it (selects, no per-lane indexing)
        int mm = 0, start = m_start[0], ln = m_Ln[0];
#pragma unroll
        for (int jm = 1; jm < kMaxMembers; ++jm) {
          if (jm < nm && k >= m_start[jm]) {
            mm = jm;
            start = m_start[jm];
            ln = m_Ln[jm];
          }
        }
        j = P + (k - start);
        e_mem = mm;
        e_L = ln >> 1;
        e_new = lane < cnt && j == new_block(ln);
      }
      e_id = ptr.block_tables[size_t(s0 + (e_mem < 0 ? 0 : e_mem)) * p.MB + j];
      e_j = j;
      e_Lm = e_L * 16 + e_mem + 1;
    }
    auto rd = [&](int v, int jj) { return __builtin_amdgcn_readlane(v, jj); };
    auto id_at = [&](int jj) {
      return first && jj == 0 ? id0 : first && jj == 1 ? id1 : rd(e_id, jj);
    };
    auto tb_of = [&](int jj) { return rd(e_j, jj) * kBlockSize; };
    auto L_of = [&](int jj) { return rd(e_Lm, jj) >> 4; };
    auto mem_of = [&](int jj) { return (rd(e_Lm, jj) & 15) - 1; };
    // the row mask of element jj: every row for a prefix block, else the
    // rows of its member
    auto act_of = [&](int jj) {
      const int mem = mem_of(jj);
      return row_ok && (mem < 0 || mem == member);
    };
    const uint64_t newmask = __builtin_amdgcn_ballot_w64(e_new);
    const auto is_new = [&](int jj) { return ((newmask >> jj) & 1ull) != 0; };
    if constexpr (kStaged) {
      constexpr int kQ = int(kTileBytes) / 1024;       // copy instructions per tile
      uint8_t* wbuf = smem + wid * kWaveLds;
      const size_t dma_lane = size_t(kvh) * kTileBytes + size_t(lane) * 16;
      auto issue = [&](int phys, int stage) {
        const size_t off = size_t(valid(phys) ? phys : 0) * block_stride + dma_lane;
        uint8_t* sb = wbuf + stage * 2 * int(kTileBytes);
#pragma unroll
        for (int r = 0; r < kQ; ++r)
          __builtin_amdgcn_global_load_lds(ptr.kcache + off + r * 1024,
                                           (lds_void_t*)(sb + r * 1024), 16, 0, kDmaPrefix);
#pragma unroll
        for (int r = 0; r < kQ; ++r)
          __builtin_amdgcn_global_load_lds(ptr.vcache + off + r * 1024,
                                           (lds_void_t*)(sb + kTileBytes + r * 1024), 16, 0,
                                           kDmaPrefix);
      };
      const uint32_t kt0 = lds_address(wbuf) + kt_lane_offset<CDT>(kq, n);
      const uint32_t v0 = lds_address(wbuf + kTileBytes + (n * kBlockSize + 4 * kq) * E);
      issue(id_at(0), 0);
      if (first) load_q();                             // behind the first tile
      for (int jj = 0; jj < cnt; ++jj) {
        const int st = jj & 1;
        if (jj + 1 < cnt) {
          issue(id_at(jj + 1), st ^ 1);
          wait_vmem<2 * kQ>();                           // element jj's stage has landed
        } else {
          wait_vmem<0>();
        }
        const int bid = id_at(jj);
        if (valid(bid)) {
          u32x2_t kraw[NC / 2];
          Raw vr[NC];
          const uint32_t so = st * 2 * uint32_t(kTileBytes);
          if (is_new(jj)) {
            // the new token into the staged tile (row d at d * 16 bytes),
            // then the tile back to the caches, 1 KiB per instruction
            const int o_new = (L_of(jj) - 1) & (kBlockSize - 1);
            const auto nr = new_rows(mem_of(jj));
            uint8_t* sb = wbuf + so;
            for (int d = lane; d < D; d += 64) {
              sb[d * kBlockSize + o_new] =
                  uint8_t(new_token_bits<QDT, CDT>(p.knew + nr.first, d, p.enc_k));
              sb[kTileBytes + d * kBlockSize + o_new] =
                  uint8_t(new_token_bits<QDT, CDT>(p.vnew + nr.second, d, p.enc_v));
            }
            const size_t goff = size_t(bid) * block_stride + dma_lane;
#pragma unroll
            for (int r = 0; r < kQ; ++r) {
              *reinterpret_cast<u32x4_t*>(const_cast<uint8_t*>(ptr.kcache) + goff + r * 1024) =
                  *reinterpret_cast<const u32x4_t*>(sb + r * 1024 + lane * 16);
              *reinterpret_cast<u32x4_t*>(const_cast<uint8_t*>(ptr.vcache) + goff + r * 1024) =
                  *reinterpret_cast<const u32x4_t*>(sb + kTileBytes + r * 1024 + lane * 16);
            }
            wait_vmem<0>();                              // counts stay exact for the copies
          }
          StagedKtV<CDT, NC>::read(kt0 + so, v0 + so, kraw, vr);
          short4_t kt[NC];
          kt_operands<QDT, CDT, NC>(kraw, kt);
          block(kt, vr, tb_of(jj), L_of(jj), act_of(jj));
        }
      }
    } else {
      // 16-bit caches: K tiles are copied into a two-stage LDS ring of the
      // wave by the direct global->LDS load (1 KiB per instruction) and read
      // back transposed, so no MFMA transposes and conversions are spent on
      // them (this walk repeats its per-tile work for each 16-row tile of a
      // group, so that work showed: an ablation without any tile loads took
      // 43 of the call's 54 us); V tiles load into registers, double-buffered.
      // Element e's operations are its kQ copies, then its NC V loads; before
      // element jj is computed only element jj + 1's are still allowed in
      // flight (loads complete in issue order).
      constexpr int kQ = int(kTileBytes) / 1024;       // copy instructions per K tile
      static_assert(2 * kTileBytes <= size_t(kWaveLds), "two K stages per wave");
      uint8_t* wbuf = smem + wid * kWaveLds;
      const size_t dma_lane = size_t(kvh) * kTileBytes + size_t(lane) * 16;
      const uint32_t kt0 = lds_address(wbuf) + kt_lane_offset<CDT>(kq, n);
      auto issue = [&](int phys, int stage, Raw (&vr)[NC]) {
        const size_t off = size_t(valid(phys) ? phys : 0) * block_stride;
        uint8_t* sb = wbuf + stage * int(kTileBytes);
#pragma unroll
        for (int r = 0; r < kQ; ++r)
          __builtin_amdgcn_global_load_lds(ptr.kcache + off + dma_lane + r * 1024,
                                           (lds_void_t*)(sb + r * 1024), 16, 0, kDmaPrefix);
#pragma unroll
        for (int c = 0; c < NC; ++c) vr[c] = load_raw<CDT>(vbase + off + c * kChunkBytes);
      };
      auto run = [&](int id, int jj, int stage, Raw (&vr)[NC]) {
        if (valid(id)) {
          const uint32_t so = uint32_t(stage) * uint32_t(kTileBytes);
          if (is_new(jj)) {
            // the whole tile back to the caches: K from its stage, V from
            // registers
            const size_t goff = size_t(id) * block_stride;
#pragma unroll
            for (int r = 0; r < kQ; ++r)
              *reinterpret_cast<u32x4_t*>(const_cast<uint8_t*>(ptr.kcache) + goff + dma_lane +
                                          r * 1024) =
                  *reinterpret_cast<const u32x4_t*>(wbuf + so + r * 1024 + lane * 16);
#pragma unroll
            for (int c = 0; c < NC; ++c)
              *reinterpret_cast<Raw*>(const_cast<uint8_t*>(vbase) + goff + c * kChunkBytes) = vr[c];
          }
          // K^T in two halves of chunks (fewer operand registers live)
          float4_t st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            u32x2_t kh[NC / 2];
            StagedKt16<NC / 2>::read(kt0 + so + uint32_t(hf * (NC / 2) * 512), kh);
#pragma unroll
            for (int c = 0; c < NC / 2; ++c)
              st = Mfma<QDT>::run(Mfma<QDT>::from_bits(__builtin_bit_cast(short4_t, kh[c])),
                                  qb[hf * (NC / 2) + c], st);
          }
          finish(st, vr, tb_of(jj), L_of(jj), act_of(jj));
        } else {
          // not computed, but consumed all the same
#pragma unroll
          for (int c = 0; c < NC; ++c) asm volatile("" ::"v"(vr[c]));
        }
      };
      Raw va[NC], vb[NC];
      int ia = id_at(0);
      if (is_new(0)) wait_vmem<0>();
      issue(ia, 0, va);
      if (first) load_q();                             // behind the first tile
      int jj = 0;
      for (; jj + 1 < cnt; jj += 2) {
        const int ib = id_at(jj + 1);
        if (is_new(jj + 1)) wait_vmem<0>();
        issue(ib, 1, vb);
        wait_vmem<kQ + NC>();                          // element jj (and q) has landed
        run(ia, jj, 0, va);
        if (jj + 2 < cnt) {
          const int ia2 = id_at(jj + 2);
          if (is_new(jj + 2)) wait_vmem<0>();
          issue(ia2, 0, va);
          wait_vmem<kQ + NC>();
          ia = ia2;
        } else {
          wait_vmem<0>();
        }
        run(ib, jj + 1, 1, vb);
      }
      if (jj < cnt) {
        wait_vmem<0>();
        run(ia, jj, 0, va);
      }
    }
    asm volatile("" ::"v"(e_id));                      // (the table load too, when unused)
  };
  // a wave's list is nearly always one chunk: walked outside any loop, so
  // that no loop-carried state makes the first tiles wait
  if (n_el <= 64) {
    if (n_el > 0) walk_chunk(0, n_el, true);
  } else {
    for (int c0 = 0; c0 < n_el; c0 += 64) walk_chunk(c0, (n_el - c0) < 64 ? (n_el - c0) : 64, c0 == 0);
  }
  l += xor_lane<16>(l);
  l += xor_lane<32>(l);

  // combine the waves through LDS; rows n < rows are written
  if (row_ok) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int i = 0; i < 4; ++i) c_o(wid, n, 16 * c + 4 * kq + i) = o[c][i];
    }
    if (kq == 0) {
      c_m[wid][n] = m;
      c_l[wid][n] = l;
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < rows * D; idx += 64 * NW) {
    const int hn = idx / D, d = idx % D;
    float Mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < NW; ++k) Mx = fmaxf(Mx, c_m[k][hn]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      const float wk = c_m[k][hn] == -INFINITY ? 0.f : fast_exp2(c_m[k][hn] - Mx);
      num = fmaf(wk, c_o(k, hn, d), num);
      den = fmaf(wk, c_l[k][hn], den);
    }
    QS* out = reinterpret_cast<QS*>(ptr.out) + size_t(s0 + hn / g) * p.o_stride +
              size_t(kvh * g + hn % g) * D;
    out[d] = from_f32<QDT>(den > 0.f ? num * (p.v_scale / den) : 0.f);
  }
}

// Waves per work-group of decode_group_kernel: 8 short walks per tile keep
// more tiles in flight than 4 long ones (each wave holds a whole tile's
// state, and 4 waves left the walks waiting on memory).
constexpr int kGroupWaves = 8;

template <DT QDT, DT CDT, int D>
__global__ __launch_bounds__(64 * kGroupWaves) __attribute__((amdgpu_waves_per_eu(4)))
void decode_group_kernel(DecodePtrs ptr, DecodeParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kGroupWaves * MfmaLds<CDT, D>::kWave];
  __shared__ float c_m[kGroupWaves][16], c_l[kGroupWaves][16];
  group_walk<QDT, CDT, D, kGroupWaves>(ptr, p, blockIdx.x, smem, c_m, c_l);
}

template <DT Q, DT C, int D>
hipError_t run_group(const DecodePtrs& ptr, const DecodeParams& p, hipStream_t stream) {
  const long long pairs8 = (1LL * p.G * p.Hk + 7) / 8 * 8;
  hipLaunchKernelGGL((decode_group_kernel<Q, C, D>), dim3(unsigned(pairs8 * p.gt)),
                     dim3(64 * kGroupWaves), 0, stream, ptr, p);
  return hipGetLastError();
}

template <DT Q, DT C>
hipError_t by_d_group(int D, const DecodePtrs& ptr, const DecodeParams& p, hipStream_t st) {
  return D == 64 ? run_group<Q, C, 64>(ptr, p, st) : run_group<Q, C, 128>(ptr, p, st);
}

template <DT Q, DT C, int D>
hipError_t run(const DecodePtrs& ptr, const DecodeParams& p, hipStream_t stream) {
  const long long units = 1LL * p.np_run * p.S * p.Hk;
  const dim3 grid{unsigned(units)}, block{64 * kWaves};
  if constexpr (D > 128) {
    switch (p.lbs) {
      case 3: hipLaunchKernelGGL((decode_mfma_wide_kernel<Q, C, D, 8>), grid, block, 0, stream, ptr, p); break;
      case 5: hipLaunchKernelGGL((decode_mfma_wide_kernel<Q, C, D, 32>), grid, block, 0, stream, ptr, p); break;
      default: hipLaunchKernelGGL((decode_mfma_wide_kernel<Q, C, D, 16>), grid, block, 0, stream, ptr, p);
    }
  } else {
    switch (p.lbs) {
      case 3: hipLaunchKernelGGL((decode_mfma_kernel<Q, C, D, 8>), grid, block, 0, stream, ptr, p); break;
      case 5: hipLaunchKernelGGL((decode_mfma_kernel<Q, C, D, 32>), grid, block, 0, stream, ptr, p); break;
      default: hipLaunchKernelGGL((decode_mfma_kernel<Q, C, D, 16>), grid, block, 0, stream, ptr, p);
    }
  }
  return hipGetLastError();
}

template <DT Q, DT C, int D>
hipError_t run_prefix(const DecodePtrs& ptr, const DecodeParams& p, hipStream_t stream) {
  const long long units = 1LL * p.rounds * p.G * p.npp * p.Hk;
  hipLaunchKernelGGL((decode_prefix_kernel<Q, C, D>), dim3(unsigned(units)), dim3(64 * kWaves),
                     0, stream, ptr, p);
  return hipGetLastError();
}

// head sizes: multiples of 16 up to 128, 192 and 256 for 16-bit caches, 64
// and 128 for E4M3 (whose tiles are copied 1 KiB at a time)
template <DT Q, DT C>
hipError_t by_d(int D, const DecodePtrs& ptr, const DecodeParams& p, hipStream_t st) {
  if constexpr (C == DT::FP8) {
    switch (D) {
      case 64: return run<Q, C, 64>(ptr, p, st);
      case 128: return run<Q, C, 128>(ptr, p, st);
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (D) {
      case 32: return run<Q, C, 32>(ptr, p, st);
      case 64: return run<Q, C, 64>(ptr, p, st);
      case 80: return run<Q, C, 80>(ptr, p, st);
      case 96: return run<Q, C, 96>(ptr, p, st);
      case 112: return run<Q, C, 112>(ptr, p, st);
      case 128: return run<Q, C, 128>(ptr, p, st);
      case 192: return run<Q, C, 192>(ptr, p, st);
      case 256: return run<Q, C, 256>(ptr, p, st);
      default: return hipErrorInvalidValue;
    }
  }
}

template <DT Q, DT C>
hipError_t by_d_prefix(int D, const DecodePtrs& ptr, const DecodeParams& p, hipStream_t st) {
  return D == 64 ? run_prefix<Q, C, 64>(ptr, p, st) : run_prefix<Q, C, 128>(ptr, p, st);
}

}  // namespace

hipError_t launch_decode_mfma(DT q, DT c, int D, const DecodePtrs& ptr, const DecodeParams& p,
                              hipStream_t stream) {
  if (q == DT::F16) {
    return c == DT::FP8 ? by_d<DT::F16, DT::FP8>(D, ptr, p, stream)
                        : by_d<DT::F16, DT::F16>(D, ptr, p, stream);
  }
  return c == DT::FP8 ? by_d<DT::BF16, DT::FP8>(D, ptr, p, stream)
                      : by_d<DT::BF16, DT::BF16>(D, ptr, p, stream);
}

hipError_t launch_decode_prefix(DT q, DT c, int D, const DecodePtrs& ptr, const DecodeParams& p,
                                hipStream_t stream) {
  if (q == DT::F16) {
    return c == DT::FP8 ? by_d_prefix<DT::F16, DT::FP8>(D, ptr, p, stream)
                        : by_d_prefix<DT::F16, DT::F16>(D, ptr, p, stream);
  }
  return c == DT::FP8 ? by_d_prefix<DT::BF16, DT::FP8>(D, ptr, p, stream)
                      : by_d_prefix<DT::BF16, DT::BF16>(D, ptr, p, stream);
}

hipError_t launch_decode_group(DT q, DT c, int D, const DecodePtrs& ptr, const DecodeParams& p,
                               hipStream_t stream) {
  if (q == DT::F16) {
    return c == DT::FP8 ? by_d_group<DT::F16, DT::FP8>(D, ptr, p, stream)
                        : by_d_group<DT::F16, DT::F16>(D, ptr, p, stream);
  }
  return c == DT::FP8 ? by_d_group<DT::BF16, DT::FP8>(D, ptr, p, stream)
                      : by_d_group<DT::BF16, DT::BF16>(D, ptr, p, stream);
}

}  // namespace pkv
