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
#include "device_common.h"

namespace pkv {
namespace {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

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
  // 4 E4M3 codes -> 4 f16 (exact: every E4M3 value is an f16 value)
  static __device__ __forceinline__ short4_t fp8x4(uint32_t w) {
    short4_t r;
    const auto lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
    const auto hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, true);
    r[0] = bits(lo[0]);
    r[1] = bits(lo[1]);
    r[2] = bits(hi[0]);
    r[3] = bits(hi[1]);
    return r;
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
  // 4 E4M3 codes -> 4 bf16 (exact: every E4M3 value is a bf16 value)
  static __device__ __forceinline__ short4_t fp8x4(uint32_t w) {
    short4_t r;
    const auto lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
    const auto hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, true);
    r[0] = bits(lo[0]);
    r[1] = bits(lo[1]);
    r[2] = bits(hi[0]);
    r[3] = bits(hi[1]);
    return r;
  }
};

// One lane's 4 tokens of one row of a 16-row chunk, as loaded (raw bits).
template <DT CDT> struct RawChunk { using type = short4_t; };
template <> struct RawChunk<DT::FP8> { using type = uint32_t; };

// FP8 tiles are staged through LDS instead: each lane's 4-byte operand load
// moves only 256 bytes per instruction, and those loads measured ~30% slower
// than copying the tile with the direct global->LDS load (16 bytes per lane,
// 1 KiB per instruction) and reading the operands back from LDS.  LDS reads
// of one staged K/V pair in the operand layout: chunk c of K sits 256 c bytes
// into the stage and V follows K, so the reads are ds_read2st64_b32 with
// offsets counted in 256-byte units.  The wait for their data is part of the
// same statement, so no result is used before it has arrived.
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
template <int NC> struct Fp8StagedPair;
template <> struct Fp8StagedPair<8> {
  static __device__ __forceinline__ void read(uint32_t a, uint32_t (&k)[8], uint32_t (&v)[8]) {
    u32x2_t r0, r1, r2, r3, r4, r5, r6, r7;
    asm volatile(
        "ds_read2st64_b32 %0, %8 offset0:0 offset1:1\n\t"
        "ds_read2st64_b32 %1, %8 offset0:2 offset1:3\n\t"
        "ds_read2st64_b32 %2, %8 offset0:4 offset1:5\n\t"
        "ds_read2st64_b32 %3, %8 offset0:6 offset1:7\n\t"
        "ds_read2st64_b32 %4, %8 offset0:8 offset1:9\n\t"
        "ds_read2st64_b32 %5, %8 offset0:10 offset1:11\n\t"
        "ds_read2st64_b32 %6, %8 offset0:12 offset1:13\n\t"
        "ds_read2st64_b32 %7, %8 offset0:14 offset1:15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6),
          "=&v"(r7)
        : "v"(a)
        : "memory");
    const u32x2_t kk[4] = {r0, r1, r2, r3}, vv[4] = {r4, r5, r6, r7};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      k[2 * i] = kk[i].x;
      k[2 * i + 1] = kk[i].y;
      v[2 * i] = vv[i].x;
      v[2 * i + 1] = vv[i].y;
    }
  }
};
template <> struct Fp8StagedPair<4> {
  static __device__ __forceinline__ void read(uint32_t a, uint32_t (&k)[4], uint32_t (&v)[4]) {
    u32x2_t r0, r1, r2, r3;
    asm volatile(
        "ds_read2st64_b32 %0, %4 offset0:0 offset1:1\n\t"
        "ds_read2st64_b32 %1, %4 offset0:2 offset1:3\n\t"
        "ds_read2st64_b32 %2, %4 offset0:4 offset1:5\n\t"
        "ds_read2st64_b32 %3, %4 offset0:6 offset1:7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
        : "v"(a)
        : "memory");
    k[0] = r0.x;
    k[1] = r0.y;
    k[2] = r1.x;
    k[3] = r1.y;
    v[0] = r2.x;
    v[1] = r2.y;
    v[2] = r3.x;
    v[3] = r3.y;
  }
};

// Wait until at most N vector-memory operations of this wave are outstanding
// (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
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

template <DT QDT, DT CDT, int D>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(4)))
void decode_mfma_kernel(DecodePtrs ptr, DecodeParams p) {
  using M = Mfma<QDT>;
  using QS = typename Elem<QDT>::storage;
  constexpr int E = Elem<CDT>::bytes;
  constexpr int NC = D / 16;                           // 16-row chunks per tile
  constexpr size_t kTileBytes = size_t(D) * kBlockSize * E;

  // FP8 caches: two K/V stages per wave in LDS (two stages at 4 waves per
  // SIMD measured faster than three or four stages at lower occupancy).
  // After the walk the same bytes hold the wave's partial O[h][d] for the
  // combine.
  constexpr bool kStaged = CDT == DT::FP8;
  constexpr int kStages = 2;
  constexpr int kCombineLds = 16 * D * 4;
  constexpr int kStageLds = kStaged ? kStages * 2 * int(kTileBytes) : 0;
  constexpr int kWaveLds = kStageLds > kCombineLds ? kStageLds : kCombineLds;
  static_assert(kTileBytes % 1024 == 0, "a tile is copied 1 KiB per instruction");
  __shared__ __attribute__((aligned(16))) uint8_t smem[kWaves * kWaveLds];
  auto c_o = [&](int w, int hn, int d) -> float& {
    return reinterpret_cast<float*>(smem + w * kWaveLds)[hn * D + d];
  };
  __shared__ float c_m[kWaves][16], c_l[kWaves][16];

  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int n = lane & 15;
  const int kq = lane >> 4;
  // work items in id order, KV head fastest (dealt round-robin to the XCDs);
  // highest partition index first and sequences longest-first, as in the
  // VALU kernel
  const int unit = blockIdx.x;
  const int kvh = unit % p.Hk;
  const int part = (p.np - 1) - unit / (p.Hk * p.S);
  const int s = longest_first_sequence(part, (unit / p.Hk) % p.S, p.bpp, ptr.context_lens, p.S,
                                       p.MB);
  if (s < 0) return;                                   // empty work item: the group leaves

  const int l_raw = ptr.context_lens[s];
  const int nb = blocks_of(l_raw, p.MB);
  const int L = l_raw > 0 ? (l_raw < nb * kBlockSize ? l_raw : nb * kBlockSize) : 0;
  const int nparts = nb == 0 ? 1 : (nb + p.bpp - 1) / p.bpp;

  const int g = p.g;
  const int h = kvh * g + n;                            // this lane's query head (if n < g)
  const bool head_ok = n < g;

  // B operand of S^T = K^T Q^T: Q[h = n][d = 16 c + 4 kq + i]
  typename M::vec qb[NC];
  {
    const QS* q = reinterpret_cast<const QS*>(ptr.query) + (size_t(s) * p.H + (head_ok ? h : 0)) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      short4_t v = *reinterpret_cast<const short4_t*>(q + 16 * c + 4 * kq);
      if (!head_ok) v = short4_t{0, 0, 0, 0};
      qb[c] = M::from_bits(v);
    }
  }
  // identity B operand: B[k = 4 kq + i][n] = (4 kq + i == n)
  typename M::vec ident;
  {
    short4_t v;
    const short one = M::bits(1.0f);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (4 * kq + i == n) ? one : short(0);
    ident = M::from_bits(v);
  }

  // the sequence's blocks are split into nparts nearly equal runs, and the
  // work-group's run among its waves the same way
  const int pj0 = (part * nb) / nparts;
  const int pj1 = ((part + 1) * nb) / nparts;
  const int j0 = pj0 + (wid * (pj1 - pj0)) / kWaves;
  const int j1 = pj0 + ((wid + 1) * (pj1 - pj0)) / kWaves;
  const int32_t* bt = ptr.block_tables + size_t(s) * p.MB;
  // lane's 4 tokens (4 kq .. 4 kq + 3) of row n of each chunk
  const size_t lane_off = size_t(kvh) * kTileBytes + (size_t(n) * kBlockSize + 4 * kq) * E;
  const size_t block_stride = size_t(p.Hk) * kTileBytes;
  constexpr size_t kChunkBytes = size_t(16) * kBlockSize * E;
  const uint8_t* kbase = ptr.kcache + lane_off;
  const uint8_t* vbase = ptr.vcache + lane_off;

  float m = -INFINITY, l = 0.f;
  float4_t o[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) o[c] = float4_t{0.f, 0.f, 0.f, 0.f};
  const float4_t zero4 = {0.f, 0.f, 0.f, 0.f};

  using Raw = typename RawChunk<CDT>::type;
  auto valid = [&](int phys) { return static_cast<unsigned>(phys) < static_cast<unsigned>(p.NB); };
  auto load_k = [&](int phys, Raw (&kr)[NC]) {
    const size_t off = size_t(valid(phys) ? phys : 0) * block_stride;
#pragma unroll
    for (int c = 0; c < NC; ++c) kr[c] = load_raw<CDT>(kbase + off + c * kChunkBytes);
  };
  auto load_v = [&](int phys, Raw (&vr)[NC]) {
    const size_t off = size_t(valid(phys) ? phys : 0) * block_stride;
#pragma unroll
    for (int c = 0; c < NC; ++c) vr[c] = load_raw<CDT>(vbase + off + c * kChunkBytes);
  };

  // one block of 16 tokens: scores, online softmax, weighted sum
  auto block = [&](const Raw (&kraw)[NC], const Raw (&vraw)[NC], int tb) {
    short4_t kr[NC], vr[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      kr[c] = to_operand<QDT, CDT>(kraw[c]);
      vr[c] = to_operand<QDT, CDT>(vraw[c]);
    }
    if (tb + kBlockSize > L) {          // zero tail tokens: they may hold NaN
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (tb + 4 * kq + i >= L) {
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            kr[c][i] = 0;
            vr[c][i] = 0;
          }
        }
      }
    }

    // scores S^T[t][h], accumulated over the NC chunks of head_size
    float4_t st = zero4;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const float4_t tt = M::run(M::from_bits(kr[c]), ident, zero4);   // K[4kq+i][n]
      short4_t tb16;
#pragma unroll
      for (int i = 0; i < 4; ++i) tb16[i] = M::bits(tt[i]);             // exact
      st = M::run(M::from_bits(tb16), qb[c], st);
    }

    // online softmax for head n over tokens 4 kq + i
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = (tb + 4 * kq + i < L) ? st[i] * p.qk_scale : -INFINITY;
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
      ph[i] = M::bits(pr);
      const float rest = pr - M::value(ph[i]);
      pl[i] = M::bits(rest);
      psum += M::value(ph[i]) + M::value(pl[i]);
    }
    l = fmaf(l, alpha, psum);

    // rescale the running sums only when some head's maximum moved (after
    // the first few blocks it rarely does); the test is wave-uniform
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
      for (int c = 0; c < NC; ++c) o[c] = o[c] * alpha;
    }
    // O^T[d][h] = sum_t V[d][t] P^T[t][h]
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float4_t acc = M::run(M::from_bits(vr[c]), M::from_bits(ph), o[c]);
      o[c] = M::run(M::from_bits(vr[c]), M::from_bits(pl), acc);
    }
  };

  // Block walk: ids fetched 64 at a time and read with readlane.  Loads are
  // unconditional (an id outside the pool reads block 0; its compute is
  // skipped).
  if constexpr (kStaged) {
    // Block j+1's K and V tiles are copied into the other LDS stage while
    // block j is computed; each wave uses only its own kWaveLds bytes.
    typedef __attribute__((address_space(3))) void lds_void_t;
    typedef __attribute__((address_space(3))) uint8_t lds_u8_t;
    constexpr int kQ = int(kTileBytes) / 1024;         // copy instructions per tile
    uint8_t* wbuf = smem + wid * kWaveLds;
    const size_t dma_lane = size_t(kvh) * kTileBytes + size_t(lane) * 16;
    auto issue = [&](int phys, int stage) {
      const size_t off = size_t(valid(phys) ? phys : 0) * block_stride + dma_lane;
      uint8_t* sb = wbuf + stage * 2 * int(kTileBytes);
#pragma unroll
      for (int r = 0; r < kQ; ++r)
        __builtin_amdgcn_global_load_lds(ptr.kcache + off + r * 1024,
                                         (lds_void_t*)(sb + r * 1024), 16, 0, 0);
#pragma unroll
      for (int r = 0; r < kQ; ++r)
        __builtin_amdgcn_global_load_lds(ptr.vcache + off + r * 1024,
                                         (lds_void_t*)(sb + kTileBytes + r * 1024), 16, 0, 0);
    };
    // LDS address of this lane's operand bytes in stage 0
    const uint32_t rd0 = static_cast<uint32_t>(
        reinterpret_cast<size_t>((lds_u8_t*)(wbuf + n * kBlockSize + 4 * kq)));
    for (int c0 = j0; c0 < j1; c0 += 64) {
      const int cnt = (j1 - c0) < 64 ? (j1 - c0) : 64;
      const int my_id = lane < cnt ? bt[c0 + lane] : 0;
      auto id_at = [&](int jj) { return __builtin_amdgcn_readlane(my_id, jj); };
      issue(id_at(0), 0);
      for (int jj = 0; jj < cnt; ++jj) {
        const int st = jj & 1;
        if (jj + 1 < cnt) {
          issue(id_at(jj + 1), st ^ 1);
          wait_vmem<2 * kQ>();                           // block jj's stage has landed
        } else {
          wait_vmem<0>();
        }
        const int id = id_at(jj);
        if (valid(id)) {
          Raw kr[NC], vr[NC];
          Fp8StagedPair<NC>::read(rd0 + st * 2 * uint32_t(kTileBytes), kr, vr);
          block(kr, vr, (c0 + jj) * kBlockSize);
        }
      }
    }
  } else {
  // K tiles are double-buffered in registers (block j+1's K is in flight
  // while block j is computed) and block j's V is issued just before block
  // j+1's K, so that the weighted sum waits for V(j) only.
  for (int c0 = j0; c0 < j1; c0 += 64) {
    const int cnt = (j1 - c0) < 64 ? (j1 - c0) : 64;
    const int my_id = lane < cnt ? bt[c0 + lane] : 0;
    auto id_at = [&](int jj) { return __builtin_amdgcn_readlane(my_id, jj); };
    Raw ka[NC], kb[NC], vc[NC];
    int ia = id_at(0);
    load_k(ia, ka);
    int jj = 0;
    for (; jj + 1 < cnt; jj += 2) {
      const int ib = id_at(jj + 1);
      load_v(ia, vc);
      load_k(ib, kb);
      if (valid(ia)) block(ka, vc, (c0 + jj) * kBlockSize);
      const int ia2 = id_at(jj + 2 < cnt ? jj + 2 : jj + 1);
      load_v(ib, vc);
      load_k(ia2, ka);
      if (valid(ib)) block(kb, vc, (c0 + jj + 1) * kBlockSize);
      ia = ia2;
    }
    if (jj < cnt) {
      load_v(ia, vc);
      if (valid(ia)) block(ka, vc, (c0 + jj) * kBlockSize);
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
    if (nparts == 1) {
      QS* out = reinterpret_cast<QS*>(ptr.out) + (size_t(s) * p.H + hq) * D;
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

template <DT Q, DT C, int D>
hipError_t run(const DecodePtrs& ptr, const DecodeParams& p, hipStream_t stream) {
  const long long units = 1LL * p.np * p.S * p.Hk;
  hipLaunchKernelGGL((decode_mfma_kernel<Q, C, D>), dim3(unsigned(units)), dim3(64 * kWaves), 0,
                     stream, ptr, p);
  return hipGetLastError();
}

template <DT Q, DT C>
hipError_t by_d(int D, const DecodePtrs& ptr, const DecodeParams& p, hipStream_t st) {
  return D == 64 ? run<Q, C, 64>(ptr, p, st) : run<Q, C, 128>(ptr, p, st);
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

}  // namespace pkv
