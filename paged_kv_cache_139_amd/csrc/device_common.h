// Device helpers shared by the gfx950 kernels: element formats, wave-level
// lane exchanges, the E4M3FN encoder and the XCD-aware work-item mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace pkv {

// ---------------------------------------------------------------------------
// element formats
// ---------------------------------------------------------------------------
template <DT T> struct Elem;
template <> struct Elem<DT::F32>  { using storage = float;    static constexpr int bytes = 4; };
template <> struct Elem<DT::F16>  { using storage = _Float16; static constexpr int bytes = 2; };
template <> struct Elem<DT::BF16> { using storage = uint16_t; static constexpr int bytes = 2; };
template <> struct Elem<DT::FP8>  { using storage = uint8_t;  static constexpr int bytes = 1; };

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

template <DT T>
__device__ __forceinline__ float load_f32(const typename Elem<T>::storage* p) {
  if constexpr (T == DT::F32) return *p;
  else if constexpr (T == DT::F16) return static_cast<float>(*p);
  else if constexpr (T == DT::BF16) return bf16_bits_to_f32(*p);
  else return 0.f;
}

// float -> storage, rounding to nearest even (hardware converts on gfx950).
template <DT T>
__device__ __forceinline__ typename Elem<T>::storage from_f32(float x) {
  if constexpr (T == DT::F32) return x;
  else if constexpr (T == DT::F16) return static_cast<_Float16>(x);
  else return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// Two E4M3FN codes (the low or the high 16 bits of `w`) -> two floats.
template <bool HI>
__device__ __forceinline__ void fp8x2_to_f32(uint32_t w, float& a, float& b) {
  auto f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, HI);
  a = f[0];
  b = f[1];
}

// The 16-byte segment `u` holds 16/bytes(T) consecutive tokens of one row
// (one head_size index) of a cache block; expand them to float.
template <DT T, int N>
__device__ __forceinline__ void segment_to_f32(const uint4& u, float (&out)[N]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  if constexpr (T == DT::F32) {
    static_assert(N == 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(w[i]);
  } else if constexpr (T == DT::F16) {
    static_assert(N == 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w[i])));
      out[2 * i + 1] =
          static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w[i] >> 16)));
    }
  } else if constexpr (T == DT::BF16) {
    static_assert(N == 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    static_assert(N == 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fp8x2_to_f32<false>(w[i], out[4 * i], out[4 * i + 1]);
      fp8x2_to_f32<true>(w[i], out[4 * i + 2], out[4 * i + 3]);
    }
  }
}

// ---------------------------------------------------------------------------
// KV tile loads.  The caches are read once per decode call, so the loads are
// marked nontemporal (the `nt` bit): measured about 5% more gather bandwidth
// than plain loads on MI355X for 4 KiB tiles at random places.
// ---------------------------------------------------------------------------
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 load_nt16(const uint8_t* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return uint4{v[0], v[1], v[2], v[3]};
}
__device__ __forceinline__ u32x2_t load_nt8(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
}

// ---------------------------------------------------------------------------
// lane exchanges inside a 64-wide wavefront: value of lane (lane ^ MASK)
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <int PATTERN>
__device__ __forceinline__ float swizzle(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), PATTERN));
}

template <int MASK>
__device__ __forceinline__ float xor_lane(float v) {
  if constexpr (MASK == 1) {
    return dpp_mov<0xB1>(v);                      // quad_perm [1,0,3,2]
  } else if constexpr (MASK == 2) {
    return dpp_mov<0x4E>(v);                      // quad_perm [2,3,0,1]
  } else if constexpr (MASK == 8) {
    return dpp_mov<0x128>(v);                     // row_ror:8 == xor 8 inside a 16-lane row
  } else if constexpr (MASK == 4 || MASK == 16) {
    return swizzle<0x1F | (MASK << 10)>(v);       // bitmask mode, xor within 32 lanes
  } else {
    static_assert(MASK == 32);
    const int src = (static_cast<int>(__lane_id()) ^ 32) << 2;
    return __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(v)));
  }
}

// ---------------------------------------------------------------------------
// fast exp2 (hardware v_exp_f32; exp2(-inf) = 0)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// E4M3FN encoder in integer arithmetic: nearest, ties to even, saturating,
// NaN -> 0x7F with the sign, sign of zero kept (OCP 8-bit FP, E4M3 table).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t f32_to_e4m3(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu | sign;               // NaN
  if (a >= 0x43e00000u) return 0x7eu | sign;              // >= 448 (and inf): saturate
  if (a < 0x3c800000u) {                                  // below 2^-6: subnormal grid k * 2^-9
    const float k = __builtin_rintf(__uint_as_float(a) * 512.0f);   // exact scaling, RNE
    return static_cast<uint32_t>(k) | sign;               // k == 8 is the smallest normal
  }
  const uint32_t exp = (a >> 23) - 120u;                  // unbiased + 7, in 1..15
  const uint32_t mant = a & 0x7fffffu;
  const uint32_t keep = mant >> 20;
  const uint32_t rest = mant & 0xfffffu;
  uint32_t code = (exp << 3) | keep;
  if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) code += 1u;   // carry is correct
  return code | sign;
}

// The cache bits of element d of a new token's row (decode with append: the
// writer's conversion, a bit copy or E4M3 of one float32 division by the
// scale, as reshape_and_cache stores it).
template <DT SRC, DT CDT>
__device__ __forceinline__ uint32_t new_token_bits(const uint8_t* row, int d, float scale) {
  using SS = typename Elem<SRC>::storage;
  if constexpr (SRC == CDT) {
    if constexpr (sizeof(SS) == 4) return reinterpret_cast<const uint32_t*>(row)[d];
    else return reinterpret_cast<const uint16_t*>(row)[d];
  } else {
    return f32_to_e4m3(__fdiv_rn(load_f32<SRC>(reinterpret_cast<const SS*>(row) + d), scale));
  }
}

// ---------------------------------------------------------------------------
// Decode work-groups: kWaves waves split a work item's blocks and merge their
// partial results through LDS.
// ---------------------------------------------------------------------------
constexpr int kWaves = 4;

// Longest-first order of the work items (both decode kernels).  Work-groups
// are handed out in id order; giving the first ids to the largest items (the
// classic longest-processing-time rule) leaves only small ones for the end of
// the launch, where the machine drains (measured 7% on the LLaMA-7B-shaped
// batch).  Items are ordered by partition index, highest first (a sequence's
// later partitions exist only when it is long), then by the sequence's tile
// count, most first, then by sequence index.
//
// Item ids are dense: with A(p) the number of sequences with more than p * bpp
// tiles (those that have a partition p; A(0) = S), the first A(np - 1) ids
// are partition np - 1, the next A(np - 2) partition np - 2, and so on.  The
// launch is sized for np * S items, so the ids past the last item, which exit
// at once, come at the end of the launch instead of occupying the machine at
// its start.  A count A(p) is one ballot per 64 sequences.  The r-th sequence
// of a partition is found by a binary search on the tile count v (how many
// sequences have at least v tiles) and a pick among the sequences with
// exactly v tiles.  The first wave of each work-group computes this from
// context_lens (identically in every work-group) and hands it to the others
// through LDS: the search runs on the scalar unit, which all waves of a
// compute unit share, and 16 waves each searching kept it busy for about 5 us
// at the start of every wave.  Batches of more than 64 * kOrderChunks
// sequences keep index order.
constexpr int kOrderChunks = 16;

// Tokens of a sequence that the decode reads: context_len clamped to
// [0, cap], cap = max_num_blocks_per_seq * BLOCK_SIZE.  The decode kernels
// walk them in tiles of kTileTokens (= 16) tokens; with BLOCK_SIZE 16 a tile
// is a block.
constexpr int kTileTokens = 16;
__device__ __forceinline__ int tokens_of(int l_raw, int cap) {
  return l_raw < 0 ? 0 : (l_raw < cap ? l_raw : cap);
}
__device__ __forceinline__ int tiles_of(int l_raw, int cap) {
  return (tokens_of(l_raw, cap) + kTileTokens - 1) / kTileTokens;
}

__device__ __forceinline__ int popc64(uint64_t m) { return __builtin_popcountll(m); }

// Reads of wave-uniform addresses through the scalar data cache (loads only):
// they do not queue behind the tile loads that fill the vector memory path.
typedef const int32_t __attribute__((address_space(4)))* scalar_i32_ptr;
__device__ __forceinline__ scalar_i32_ptr scalar_ptr(const int32_t* p) {
  return (scalar_i32_ptr)p;
}

// Shared-prefix batches: the prefix length in blocks of sequence s's group
// (the last group whose first sequence is <= s), clamped to [0, MB].
__device__ __forceinline__ int group_prefix_blocks(int s, const DecodeParams& p) {
  int lo = 0, hi = p.G - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.group_starts[mid] <= s) lo = mid;
    else hi = mid - 1;
  }
  const int P = p.group_prefix[lo];
  return P < 0 ? 0 : (P > p.MB ? p.MB : P);
}

// The search over NCH chunks of 64 sequences (NCH a compile-time count, so
// that the chunk loops are straight-line code: the search runs on the scalar
// unit, which the waves of a compute unit share).
template <int NCH>
__device__ __forceinline__ int longest_first_in(int q, int np, int bpp,
                                                const int32_t* __restrict__ lens, int S,
                                                int cap, int& part, int& len) {
  const int lane = static_cast<int>(__lane_id());
  const int MB = (cap + kTileTokens - 1) / kTileTokens;    // most tiles of a sequence
  // All chunks' lengths are requested before any is used, so that they arrive
  // in one memory round trip.  Lanes past S read lens[S - 1] and get the key -1.
  int key[NCH], raw[NCH];
  {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int t = 64 * c + lane;
      raw[c] = lens[t < S ? t : S - 1];
    }
#pragma unroll
    for (int c = 0; c < NCH; ++c) key[c] = (64 * c + lane < S) ? tiles_of(raw[c], cap) : -1;
  }
  auto count_ge = [&](int v) {                   // sequences with at least v >= 1 blocks
    int n = 0;                                   // (the keys -1 never count)
#pragma unroll
    for (int c = 0; c < NCH; ++c) n += popc64(__builtin_amdgcn_ballot_w64(key[c] >= v));
    return n;
  };
  int r = q;
  part = np - 1;
  for (; part > 0; --part) {                     // skip the partitions before item q's
    const int a = count_ge(part * bpp + 1);
    if (r < a) break;
    r -= a;
  }
  if (part == 0 && r >= S) return -1;            // past the last item
  int lo = 0, hi = MB;                           // largest v with count_ge(v) > r
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (count_ge(mid) > r) lo = mid;
    else hi = mid - 1;
  }
  int k = r - count_ge(lo + 1);                  // position among those with lo blocks
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const uint64_t m = __builtin_amdgcn_ballot_w64(key[c] == lo);
    const int pc = popc64(m);
    if (k < pc) {
      const int below = static_cast<int>(__builtin_amdgcn_mbcnt_hi(
          static_cast<uint32_t>(m >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u)));
      const bool mine = ((m >> lane) & 1ull) && below == k;
      const uint64_t hit = __builtin_amdgcn_ballot_w64(mine);
      const int at = __builtin_ctzll(hit);
      len = __builtin_amdgcn_readlane(raw[c], at);
      return 64 * c + at;
    }
    k -= pc;
  }
  return -1;                                     // not reached
}

// Returns the sequence of item q (0 <= q < np * S) of a launch over np
// partitions, or -1 when there is no such item; part and len receive its
// partition and the sequence's context_lens entry.
__device__ __forceinline__ int longest_first_sequence(int q, int np, int bpp,
                                                      const int32_t* __restrict__ lens, int S,
                                                      int cap, int& part, int& len) {
  if (S > 64 * kOrderChunks) {                   // index order, empty items in place
    part = (np - 1) - q / S;
    const int r = q % S;
    len = lens[r];
    const int nb = tiles_of(len, cap);
    const int nparts = nb == 0 ? 1 : (nb + bpp - 1) / bpp;
    return part < nparts ? r : -1;
  }
  if (S <= 64) return longest_first_in<1>(q, np, bpp, lens, S, cap, part, len);
  if (S <= 256) return longest_first_in<4>(q, np, bpp, lens, S, cap, part, len);
  return longest_first_in<kOrderChunks>(q, np, bpp, lens, S, cap, part, len);
}

}  // namespace pkv
