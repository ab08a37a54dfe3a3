// Slot-mapped KV writer and the block-table gather.
//
// reshape_and_cache: each new token's key/value row [Hk, D] (token t's row
// at element t * key_stride / t * value_stride of the source) is stored into
// the paged caches at slot = block * BLOCK_SIZE + offset ([TGI] §4.1, the KV
// write side, bit copy or FP8 quantised write).
//
// The cache layout [NB, Hk, D, BLOCK_SIZE] puts a block's tokens next to each
// other within one head_size row, so a token's elements land BLOCK_SIZE
// elements apart.  Writing token by token therefore touches a different
// cache line with every element.  Instead, the writer looks for "octets":
// 8 consecutive input tokens whose slots are 8 consecutive offsets of one
// block, starting at an offset that is a multiple of 8 -- what a prefill or
// any run of a sequence's tokens in order produces.  An octet's 8 tokens fill
// 8 adjacent elements of every row of the block's tile, so they are stored as
// one 8-element piece per row (16 bytes for f16/bf16, 8 for E4M3, 32 for
// f32), with the octets of one block row on adjacent lanes: a store
// instruction then writes whole rows (1 KiB contiguous for f16 at BLOCK_SIZE
// 16).  Every other token (a single decode token per sequence, a partial
// block at the edge of a run) is stored element by element.
//
// Work-group: a window of input tokens x one KV head x one chunk of up to
// 256 source bytes of head_size.  The octets whose first token lies in the
// window belong to it (their last tokens may lie up to 7 tokens past its
// end); a token that is in no octet is stored element by element by the
// window that holds it.  An octet is recognised from the slots alone, so the
// two ways of storing never overlap and each token is stored once.  The
// source rows of the window (and of its 7-token tail when an octet may run
// into it) are copied to LDS (16 bytes per lane, converted to the cache
// format on the way for E4M3), and read back column-wise for the stores.
//
// Short batches (a decode step) use windows of 16 tokens at fixed places.
// Bulk writes place each window boundary at a block start: window k starts
// at the first token in [48 k, 48 k + 16) whose slot is the first of its
// block (at 48 k if there is none; window 0 at token 0), so a run of a
// sequence's tokens puts every block row into one window.  Then no row is
// written in two pieces by two work-groups (two partial lines), and no
// octet runs past the window, so the next window's first tokens are not read
// twice.  Neighbouring windows compute the shared boundary from the same
// slots, so they always agree on it.
//
// paged_kv_gather: the logical KV of one sequence through its block table
// ([L3] "SVG框架图"), bits unchanged.
#include <type_traits>

#include "device_common.h"

namespace pkv {
namespace {

constexpr int kWriterThreads = 256;
constexpr int kChunkBytes = 256;                 // source bytes of one (token, head) row chunk

// The writer's E4M3 quotient x / scale.  Every source magnitude a of one call
// is divided by the same scale s, so instead of a full IEEE division per
// element the writer uses the reciprocal r = RN(1/s) (computed once on the
// host) and one correction step: q0 = RN(a r), e = a - q0 s (exact, by an
// FMA), q = RN(q0 + e r).  With r the correctly rounded reciprocal and no
// underflow or overflow on the way, q is the correctly rounded a / s
// (Markstein's division theorem).  The host takes this path only for scales
// in [2^-60, 2^60]: then nothing underflows when a / s is large enough to
// have a nonzero E4M3 code (a / s >= 2^-11), and sources above lim =
// RN(1024 s), whose quotients saturate anyway, are divided as lim.  Checked
// against float32 division through the E4M3 codes of every finite 16-bit
// magnitude at 3515 scales.  Other scales use the IEEE division.
struct Fp8Scale {
  float s, r, lim;
};

// a / s for a >= 0 (or NaN), clamped to 448 (NaN stays NaN).
template <bool FAST>
__device__ __forceinline__ float e4m3_quotient(float a, Fp8Scale sc) {
  float q;
  if constexpr (FAST) {
    const float ac = a > sc.lim ? sc.lim : a;                  // (inf too; NaN stays)
    const float q0 = ac * sc.r;
    const float e = __builtin_fmaf(-q0, sc.s, ac);
    q = __builtin_fmaf(e, sc.r, q0);
  } else {
    q = __fdiv_rn(a, sc.s);
  }
  return q > 448.0f ? 448.0f : q;
}

// Four non-negative quotients (clamped to 448, or NaN) -> four E4M3
// magnitude codes in one word, first quotient in the low byte.  The gfx950
// conversion rounds to nearest even (subnormals included); it turns values
// above 464 into NaN codes (hence the clamp to 448) and NaN into a NaN code
// with the sign bit set whatever the NaN's sign, so the sign bits are
// cleared here and the source's signs put in by the caller.  A probe compared
// (clamp, convert, clear the sign bit, put in the sign) with the integer
// encoder f32_to_e4m3 on all 2^32 float32 bit patterns: no difference.
__device__ __forceinline__ uint32_t e4m3x4(float q0, float q1, float q2, float q3) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, w, true);
  return static_cast<uint32_t>(w) & 0x7f7f7f7fu;
}

// 8 source elements (16 or 32 bytes as loaded) -> 8 cache elements.
template <DT SRC, DT CACHE, bool FAST> struct Convert8;
template <DT T, bool FAST> struct Convert8<T, T, FAST> {
  static constexpr int kSrcWords = 2 * Elem<T>::bytes;       // 32-bit words loaded
  static __device__ __forceinline__ void run(const uint32_t* w, uint32_t* out, Fp8Scale) {
#pragma unroll
    for (int i = 0; i < kSrcWords; ++i) out[i] = w[i];
  }
};
template <DT SRC, bool FAST> struct Convert8<SRC, DT::FP8, FAST> {
  static constexpr int kSrcWords = 4;
  // |x| of the 16-bit element in the low (HI false) or high half of w
  template <bool HI>
  static __device__ __forceinline__ float magnitude(uint32_t w) {
    const uint32_t b = (HI ? w >> 16 : w) & 0x7fffu;
    if constexpr (SRC == DT::F16)
      return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
    else
      return __uint_as_float(b << 16);
  }
  static __device__ __forceinline__ void run(const uint32_t* w, uint32_t* out, Fp8Scale sc) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t lo = w[2 * i], hi = w[2 * i + 1];        // elements 4i .. 4i + 3
      const uint32_t codes = e4m3x4(e4m3_quotient<FAST>(magnitude<false>(lo), sc),
                                    e4m3_quotient<FAST>(magnitude<true>(lo), sc),
                                    e4m3_quotient<FAST>(magnitude<false>(hi), sc),
                                    e4m3_quotient<FAST>(magnitude<true>(hi), sc));
      // E4M3(x / scale) carries the sign of x (of a NaN too): bit 15 of each
      // source element to bit 7 of its code
      const uint32_t signs = ((lo >> 8) & 0x80u) | ((lo >> 16) & 0x8000u) |
                             ((hi << 8) & 0x800000u) | (hi & 0x80000000u);
      out[i] = codes | signs;
    }
  }
};

template <DT SRC, DT CACHE, int WIN, bool FAST, bool ALIGN>
__global__ __launch_bounds__(kWriterThreads) void reshape_and_cache_kernel(
    const uint8_t* __restrict__ key, const uint8_t* __restrict__ value, uint8_t* __restrict__ kc,
    uint8_t* __restrict__ vc, const int64_t* __restrict__ slots, int T, int Hk, int D, int NB,
    int lbs, long long key_stride, long long value_stride, Fp8Scale ksc, Fp8Scale vsc,
    int nchunks) {
  constexpr int ES = Elem<SRC>::bytes;
  constexpr int EC = Elem<CACHE>::bytes;
  constexpr int DC = kChunkBytes / ES;           // head_size elements per chunk
  // rows of LDS: a fixed window + its 7-token tail, rounded up; or an aligned
  // window (at most WIN - 1 tokens, or at most WIN - 16 + 7 with a tail)
  constexpr int ROWS = ALIGN ? WIN : WIN + 8;
  constexpr int kStep = WIN - 16;                // aligned windows: nominal start spacing
  static_assert(!ALIGN || WIN == 64, "an aligned window fits one wave's ballot");
  // LDS row of one token's chunk in cache format, padded by 16 bytes so that
  // the rows 8 apart that one store instruction reads sit in other banks
  constexpr int LROW = DC * EC + 16;
  constexpr int CW = 2 * EC;                     // 32-bit words of 8 cache elements
  using Conv = Convert8<SRC, CACHE, FAST>;
  static_assert(WIN % 8 == 0 && WIN <= 64, "window within one wave's ballot");

  __shared__ __align__(16) uint8_t lk[ROWS * LROW];
  __shared__ __align__(16) uint8_t lv[ROWS * LROW];
  // slots of tokens tn - 8 .. tn + kSlots - 9 (tn: the window's nominal start)
  constexpr int kSlots = ALIGN ? WIN + 32 : WIN + 16;
  __shared__ long long sslot[kSlots];
  __shared__ int sbound[2];                      // aligned windows: first token, token count
  __shared__ int sgrp[WIN / 8][4];               // octet starts by (block-row group, octet of row)
  __shared__ int sscal[WIN];                     // window positions stored element by element
  __shared__ int scount[2];                      // block-row groups, element-by-element tokens

  const int tid = threadIdx.x;
  const long long tn = 1LL * blockIdx.x * (ALIGN ? kStep : WIN);   // nominal start
  const int h = blockIdx.y / nchunks;
  const int d0 = (blockIdx.y % nchunks) * DC;
  const int dc = D - d0 < DC ? D - d0 : DC;      // elements of this chunk (a multiple of 8)
  const int pieces = dc / 8;                     // 8-element pieces per token row
  const long long bs = 1LL << lbs;
  const long long nslots = 1LL * NB << lbs;

  // slots of tokens tn - 8 .. (-1: outside [0, T) or no write)
  auto read_slots = [&]() {
    if (tid < kSlots) {
      const long long t = tn - 8 + tid;
      long long s = -1;
      if (t >= 0 && t < T) {
        s = slots[t];
        if (s < 0 || s >= nslots) s = -1;
      }
      sslot[tid] = s;
    }
  };
  // Source rows, 8 elements per lane, loaded into registers in up to two
  // phases and then put into LDS (row r of the window at r * LROW).  A phase
  // covers rows row_of(v) (relative to tn) for v < n; kLd loads per thread.
  auto load_rows = [&](auto nld, auto row_of, int n, uint32_t (*kw)[Conv::kSrcWords],
                       uint32_t (*vw)[Conv::kSrcWords]) {
    constexpr int kLd = decltype(nld)::value;
#pragma unroll
    for (int i = 0; i < kLd; ++i) {
      const int item = tid + i * kWriterThreads;
      const int v = item / pieces, pc = item % pieces;
      const long long t = tn + row_of(v);
      if (v < n && t < T) {
        const size_t off = size_t(h) * D + d0 + size_t(pc) * 8;
        const uint32_t* ks = reinterpret_cast<const uint32_t*>(key + (size_t(t) * key_stride + off) * ES);
        const uint32_t* vs = reinterpret_cast<const uint32_t*>(value + (size_t(t) * value_stride + off) * ES);
        // nontemporal: nearly every source row is read once (a bulk fill
        // took 5% less time than with cache-allocating loads)
#pragma unroll
        for (int j = 0; j < Conv::kSrcWords; j += 4) {
          const uint4 a = load_nt16(reinterpret_cast<const uint8_t*>(ks + j));
          const uint4 b = load_nt16(reinterpret_cast<const uint8_t*>(vs + j));
          kw[i][j] = a.x; kw[i][j + 1] = a.y; kw[i][j + 2] = a.z; kw[i][j + 3] = a.w;
          vw[i][j] = b.x; vw[i][j + 1] = b.y; vw[i][j + 2] = b.z; vw[i][j + 3] = b.w;
        }
      }
    }
  };
  // t0: the window's first token (as an offset from tn: so)
  auto store_rows = [&](auto nld, auto row_of, int n, int so, uint32_t (*kw)[Conv::kSrcWords],
                        uint32_t (*vw)[Conv::kSrcWords]) {
    constexpr int kLd = decltype(nld)::value;
#pragma unroll
    for (int i = 0; i < kLd; ++i) {
      const int item = tid + i * kWriterThreads;
      const int v = item / pieces, pc = item % pieces;
      const int rt = row_of(v);
      if (v < n && tn + rt < T) {
        const int r = rt - so;
        uint32_t ko[CW], vo[CW];
        Conv::run(kw[i], ko, ksc);
        Conv::run(vw[i], vo, vsc);
        uint32_t* kd = reinterpret_cast<uint32_t*>(lk + r * LROW + pc * 8 * EC);
        uint32_t* vd = reinterpret_cast<uint32_t*>(lv + r * LROW + pc * 8 * EC);
#pragma unroll
        for (int j = 0; j < CW; ++j) {
          kd[j] = ko[j];
          vd[j] = vo[j];
        }
      }
    }
  };
  constexpr int kPieces = DC / 8;
  // 1. the rows every window of the launch holds whatever its bounds: for
  //    fixed windows all of them (and the tail), for aligned ones tokens
  //    tn + 15 .. tn + kStep - 1 -- issued first, as they need no slot
  constexpr int kRowA0 = ALIGN ? 15 : 0;
  constexpr int kRowsA = ALIGN ? kStep - 15 : ROWS;
  constexpr int kLdA = (kRowsA * kPieces + kWriterThreads - 1) / kWriterThreads;
  uint32_t kwa[kLdA][Conv::kSrcWords], vwa[kLdA][Conv::kSrcWords];
  auto row_a = [](int v) { return kRowA0 + v; };
  load_rows(std::integral_constant<int, kLdA>{}, row_a, kRowsA, kwa, vwa);

  // 2. slots; for aligned windows, their bounds and the rest of their rows
  //    (tokens t0 .. tn + 14 and tn + kStep .. t0 + nrows - 1)
  read_slots();
  if (tid >= 64 && tid < 64 + WIN / 2) sgrp[(tid - 64) >> 2][(tid - 64) & 3] = -1;
  // the window: tokens tn + so .. tn + so + wlen - 1, and its source rows
  int wlen = WIN, nrows = ROWS;
  constexpr int kRowsB = ALIGN ? 30 : 0;         // (15 - so) + (so + nrows - kStep) <= 30
  constexpr int kLdB = (kRowsB * kPieces + kWriterThreads - 1) / kWriterThreads;
  uint32_t kwb[kLdB > 0 ? kLdB : 1][Conv::kSrcWords], vwb[kLdB > 0 ? kLdB : 1][Conv::kSrcWords];
  int so = 0, nb = 0;
  auto row_b = [&](int v) { return v < 15 - so ? so + v : kStep + v - (15 - so); };
  if constexpr (ALIGN) {
    __syncthreads();
    if (tid < 64) {
      // lanes 0..15: is token tn + lane a block's first?  lanes 16..31: is
      // token tn + kStep + lane - 16?  (the next window's start)
      const int at = tid < 16 ? tid : kStep + tid - 16;
      const long long sl = tid < 32 ? sslot[8 + at] : -1;
      const bool first = sl >= 0 && (sl & (bs - 1)) == 0;
      const uint64_t m = __builtin_amdgcn_ballot_w64(first);
      if (tid == 0) {
        const uint32_t lo = uint32_t(m & 0xFFFFu), hi = uint32_t((m >> 16) & 0xFFFFu);
        const long long a = blockIdx.x == 0 ? 0 : (lo ? tn + __builtin_ctz(lo) : tn);
        long long b = hi ? tn + kStep + __builtin_ctz(hi) : tn + kStep;
        const bool tail = hi == 0 && b < T;      // an octet may run past the end
        if (b > T) b = T;
        sbound[0] = int(a - tn);
        sbound[1] = int(b - a) | (tail ? 1 << 16 : 0);
      }
    }
    __syncthreads();
    so = sbound[0];
    const int lw = sbound[1];
    wlen = lw & 0xFFFF;
    nrows = wlen + ((lw >> 16) ? 7 : 0);
    const int past = so + nrows - kStep;
    nb = (15 - so) + (past > 0 ? past : 0);
    load_rows(std::integral_constant<int, kLdB>{}, row_b, nb, kwb, vwb);
  }
  // position i of the window (-8 <= i < wlen + 8) -> its slot
  auto slot_at = [&](int i) { return sslot[i + 8 + so]; };

  // 3. the rows into LDS, in cache format
  store_rows(std::integral_constant<int, kLdA>{}, row_a, kRowsA, so, kwa, vwa);
  if constexpr (ALIGN) store_rows(std::integral_constant<int, kLdB>{}, row_b, nb, so, kwb, vwb);
  __syncthreads();

  // 4. wave 0 sorts the window's tokens: octet starts (grouped by block row)
  //    and tokens in no octet
  if (tid < 64) {
    // is the token at window position i the first of an octet?
    auto octet_at = [&](int i) {                 // -8 < i < WIN + 8 - 7
      const long long s = slot_at(i);
      if (s < 0 || (s & 7) != 0) return false;
      bool ok = true;
#pragma unroll
      for (int j = 1; j < 8; ++j) ok = ok && slot_at(i + j) == s + j;
      return ok;
    };
    const int i = tid;
    const bool in_win = i < wlen;
    const long long s = in_win ? slot_at(i) : -1;
    const bool head = in_win && octet_at(i);
    // a token belongs to the octet that starts (s mod 8) positions before it
    const bool covered = s >= 0 && octet_at(i - int(s & 7));
    const bool scalar = s >= 0 && !covered;
    // a new block-row group unless the octet 8 positions back continues the row
    const bool cont = head && i >= 8 && octet_at(i - 8) && slot_at(i - 8) == s - 8 &&
                      ((s - 8) >> lbs) == (s >> lbs) && ((s & (bs - 1)) >> 3) != 0;
    const uint64_t below = (1ull << i) - 1ull;
    const uint64_t mnew = __builtin_amdgcn_ballot_w64(head && !cont);
    const uint64_t msc = __builtin_amdgcn_ballot_w64(scalar);
    if (head) {
      const int g = popc64(mnew & (below | (1ull << i))) - 1;
      sgrp[g][int((s & (bs - 1)) >> 3)] = i;
    }
    if (scalar) sscal[popc64(msc & below)] = i;
    if (tid == 0) {
      scount[0] = popc64(mnew);
      scount[1] = popc64(msc);
    }
  }
  __syncthreads();

  using CS = typename Elem<CACHE>::storage;
  CS* kcs = reinterpret_cast<CS*>(kc);
  CS* vcs = reinterpret_cast<CS*>(vc);
  const size_t head_base = size_t(h) * D + d0;

  // 5. octets: lane = (group, row d, octet of the row), the octet fastest, so
  //    that lanes side by side store one row's pieces and the next rows
  const int R = int(bs >> 3);                    // octets per block row
  const int ngroups = scount[0];
  for (int item = tid; item < ngroups * dc * R; item += kWriterThreads) {
    const int r = item % R;
    const int d = (item / R) % dc;
    const int g = item / (R * dc);
    const int i = sgrp[g][r];
    if (i < 0) continue;
    const long long s = slot_at(i);
    const size_t dst = (((size_t(s >> lbs) * Hk) * D + head_base + d) << lbs) + size_t(s & (bs - 1));
    uint32_t kp[CW], vp[CW];
#pragma unroll
    for (int j = 0; j < CW; ++j) {
      kp[j] = 0;
      vp[j] = 0;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int at = (i + k) * LROW + d * EC;
      uint32_t a, b;
      if constexpr (EC == 1) { a = lk[at]; b = lv[at]; }
      else if constexpr (EC == 2) {
        a = *reinterpret_cast<const uint16_t*>(lk + at);
        b = *reinterpret_cast<const uint16_t*>(lv + at);
      } else {
        a = *reinterpret_cast<const uint32_t*>(lk + at);
        b = *reinterpret_cast<const uint32_t*>(lv + at);
      }
      const int bit = (k * EC * 8) % 32, word = (k * EC * 8) / 32;
      kp[word] |= a << bit;
      vp[word] |= b << bit;
    }
    if constexpr (EC == 1) {
      *reinterpret_cast<uint2*>(kcs + dst) = uint2{kp[0], kp[1]};
      *reinterpret_cast<uint2*>(vcs + dst) = uint2{vp[0], vp[1]};
    } else {
#pragma unroll
      for (int j = 0; j < CW; j += 4) {
        *reinterpret_cast<uint4*>(reinterpret_cast<uint32_t*>(kcs + dst) + j) =
            uint4{kp[j], kp[j + 1], kp[j + 2], kp[j + 3]};
        *reinterpret_cast<uint4*>(reinterpret_cast<uint32_t*>(vcs + dst) + j) =
            uint4{vp[j], vp[j + 1], vp[j + 2], vp[j + 3]};
      }
    }
  }

  // 6. tokens in no octet, element by element (row d fastest)
  const int nscal = scount[1];
  for (int item = tid; item < nscal * dc; item += kWriterThreads) {
    const int d = item % dc;
    const int i = sscal[item / dc];
    const long long s = slot_at(i);
    const size_t dst = (((size_t(s >> lbs) * Hk) * D + head_base + d) << lbs) + size_t(s & (bs - 1));
    const int at = i * LROW + d * EC;
    if constexpr (EC == 1) {
      kcs[dst] = lk[at];
      vcs[dst] = lv[at];
    } else if constexpr (EC == 2) {
      reinterpret_cast<uint16_t*>(kcs)[dst] = *reinterpret_cast<const uint16_t*>(lk + at);
      reinterpret_cast<uint16_t*>(vcs)[dst] = *reinterpret_cast<const uint16_t*>(lv + at);
    } else {
      reinterpret_cast<uint32_t*>(kcs)[dst] = *reinterpret_cast<const uint32_t*>(lk + at);
      reinterpret_cast<uint32_t*>(vcs)[dst] = *reinterpret_cast<const uint32_t*>(lv + at);
    }
  }
}

template <typename W>
__global__ __launch_bounds__(256) void gather_kernel(W* __restrict__ k_out, W* __restrict__ v_out,
                                                     const W* __restrict__ kc,
                                                     const W* __restrict__ vc,
                                                     const int32_t* __restrict__ table, int L,
                                                     int Hk, int D, int NB, int lbs) {
  const long long item = 1LL * blockIdx.x * blockDim.x + threadIdx.x;
  if (item >= 1LL * L * Hk * D) return;
  const int d = int(item % D);
  const int h = int((item / D) % Hk);
  const int t = int(item / (1LL * D * Hk));
  const int phys = table[t >> lbs];
  W kv = 0, vv = 0;
  if (static_cast<unsigned>(phys) < static_cast<unsigned>(NB)) {
    const size_t at = (((size_t(phys) * Hk + h) * D + d) << lbs) + (t & ((1 << lbs) - 1));
    kv = kc[at];
    vv = vc[at];
  }
  k_out[item] = kv;
  v_out[item] = vv;
}

// Windows of at most 64 tokens, placed at block starts, for bulk writes; 16
// at fixed places for short batches such as one decode token per sequence,
// so that they still spread over many work-groups.
constexpr int kBulkWindow = 64;
constexpr int kShortWindow = 16;
constexpr int kShortTokens = 4096;

// The quotient path of E4M3 writes for a scale (see e4m3_quotient_code).
bool fast_quotient(float s) { return s >= 0x1p-60f && s <= 0x1p60f; }
Fp8Scale fp8_scale(float s) { return Fp8Scale{s, 1.0f / s, 1024.0f * s}; }

template <DT S, DT C>
hipError_t run_writer(const void* key, const void* value, void* kc, void* vc, const int64_t* slots,
                      int T, int Hk, int D, int NB, int lbs, long long kst, long long vst,
                      float ks, float vs, hipStream_t stream) {
  const int dc = kChunkBytes / Elem<S>::bytes;
  const int nchunks = (D + dc - 1) / dc;
  const bool bulk = T > kShortTokens;
  const int step = bulk ? kBulkWindow - 16 : kShortWindow;   // window spacing
  const dim3 grid(unsigned((T + step - 1) / step), unsigned(Hk * nchunks));
  auto launch = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(kWriterThreads), 0, stream,
                       static_cast<const uint8_t*>(key), static_cast<const uint8_t*>(value),
                       static_cast<uint8_t*>(kc), static_cast<uint8_t*>(vc), slots, T, Hk, D, NB,
                       lbs, kst, vst, fp8_scale(ks), fp8_scale(vs), nchunks);
  };
  if constexpr (C != DT::FP8) {                  // a bit copy: nothing to divide
    if (bulk) launch(reshape_and_cache_kernel<S, C, kBulkWindow, true, true>);
    else launch(reshape_and_cache_kernel<S, C, kShortWindow, true, false>);
  } else {                                       // the scales pick the quotient path
    const bool fast = fast_quotient(ks) && fast_quotient(vs);
    if (bulk) {
      if (fast) launch(reshape_and_cache_kernel<S, C, kBulkWindow, true, true>);
      else launch(reshape_and_cache_kernel<S, C, kBulkWindow, false, true>);
    } else {
      if (fast) launch(reshape_and_cache_kernel<S, C, kShortWindow, true, false>);
      else launch(reshape_and_cache_kernel<S, C, kShortWindow, false, false>);
    }
  }
  return hipGetLastError();
}

template <typename W>
hipError_t run_gather(void* ko, void* vo, const void* kc, const void* vc, const int32_t* table,
                      int L, int Hk, int D, int NB, int lbs, hipStream_t stream) {
  const long long items = 1LL * L * Hk * D;
  const unsigned grid = unsigned((items + 255) / 256);
  hipLaunchKernelGGL((gather_kernel<W>), dim3(grid), dim3(256), 0, stream, static_cast<W*>(ko),
                     static_cast<W*>(vo), static_cast<const W*>(kc), static_cast<const W*>(vc),
                     table, L, Hk, D, NB, lbs);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* kc, void* vc,
                                    const int64_t* slots, int T, int Hk, int D, int NB, int lbs,
                                    long long kst, long long vst, DT src, DT cache,
                                    float k_scale, float v_scale, hipStream_t stream) {
  if (cache == DT::FP8) {
    return src == DT::F16 ? run_writer<DT::F16, DT::FP8>(key, value, kc, vc, slots, T, Hk, D, NB,
                                                         lbs, kst, vst, k_scale, v_scale, stream)
                          : run_writer<DT::BF16, DT::FP8>(key, value, kc, vc, slots, T, Hk, D, NB,
                                                          lbs, kst, vst, k_scale, v_scale, stream);
  }
  switch (src) {
    case DT::F32:
      return run_writer<DT::F32, DT::F32>(key, value, kc, vc, slots, T, Hk, D, NB, lbs, kst, vst,
                                          1.f, 1.f, stream);
    case DT::F16:
      return run_writer<DT::F16, DT::F16>(key, value, kc, vc, slots, T, Hk, D, NB, lbs, kst, vst,
                                          1.f, 1.f, stream);
    default:
      return run_writer<DT::BF16, DT::BF16>(key, value, kc, vc, slots, T, Hk, D, NB, lbs, kst,
                                            vst, 1.f, 1.f, stream);
  }
}

hipError_t launch_gather(void* k_out, void* v_out, const void* kc, const void* vc,
                         const int32_t* table, int L, int Hk, int D, int NB, int lbs, DT cache,
                         hipStream_t stream) {
  switch (dt_bytes(cache)) {
    case 4: return run_gather<uint32_t>(k_out, v_out, kc, vc, table, L, Hk, D, NB, lbs, stream);
    case 2: return run_gather<uint16_t>(k_out, v_out, kc, vc, table, L, Hk, D, NB, lbs, stream);
    default: return run_gather<uint8_t>(k_out, v_out, kc, vc, table, L, Hk, D, NB, lbs, stream);
  }
}

}  // namespace pkv
