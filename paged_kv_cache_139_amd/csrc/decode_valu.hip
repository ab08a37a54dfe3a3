// Paged decode attention, one query head per wavefront, on the vector ALUs.
//
// Used when one query head reads each KV head (multi-head attention), and for
// every float32 case.  Work item = (partition, sequence, query head); one
// 64-lane wavefront per work item walks the partition's logical blocks
// through the block table ([L3] "注意力计算的'分页'实现"; [TGI] §4.3) and keeps an
// online softmax; partitions are merged afterwards by merge.hip ([TGI] §4.1,
// V2 partitions + reduction).
//
// Lane layout.  A block's K (or V) tile for one head is head_size rows of
// BLOCK_SIZE tokens, token fastest ([TGI] §4.2).  The walk takes tiles of TT
// tokens: 32 for 16-bit and E4M3 caches at BLOCK_SIZE 16 (two consecutive
// blocks) and 32 (one block), 16 otherwise.  Lane = (row r, segment seg)
// holds 16 bytes = TPS = 16 / E tokens of one row (E = element bytes); a
// tile row is NSEG = TT * E / 16 segments, so one load instruction covers
// R = 64 / NSEG rows (1 KiB: whole block rows, or 512 contiguous bytes of
// each block of a pair) and NL = head_size / R loads cover a tile.  The query
// element of each row a lane touches is held in a register for the whole
// partition.
//
// Dot products reduce over rows, i.e. across the R lanes of a segment: a
// reduce-scatter over row-lane bits R/2 .. SH (SH = 64 / TT) leaves each lane
// with one token (index r / SH), then an all-reduce over the bits below SH
// (DPP permutes).  Each segment keeps its own softmax state (max, sum) so the
// exponentials of a segment never need a cross-segment max; segments are
// combined once at the end of the partition.  Probabilities reach the PV
// lanes through LDS.
#include "device_common.h"

namespace pkv {
namespace {

template <int MASK, int N>
__device__ __forceinline__ void reduce_scatter(float* v, int r) {
  if constexpr (N > 1) {
    constexpr int HALF = N / 2;
    const bool upper = (r & MASK) != 0;
#pragma unroll
    for (int k = 0; k < HALF; ++k) {
      const float keep = upper ? v[k + HALF] : v[k];
      const float send = upper ? v[k] : v[k + HALF];
      v[k] = keep + xor_lane<MASK>(send);
    }
    reduce_scatter<MASK / 2, HALF>(v, r);
  }
}

// max over lanes that differ in row-lane bits 4 .. R/2 (same segment)
template <int MASK, int R>
__device__ __forceinline__ float seg_max(float v) {
  if constexpr (MASK < R) {
    return seg_max<MASK * 2, R>(fmaxf(v, xor_lane<MASK>(v)));
  } else {
    return v;
  }
}

template <int MASK, int R>
__device__ __forceinline__ float seg_sum(float v) {
  if constexpr (MASK < R) {
    return seg_sum<MASK * 2, R>(v + xor_lane<MASK>(v));
  } else {
    return v;
  }
}

// Direct global->LDS load of 4 bytes per lane (lane i's bytes to lds + 4 i;
// lds wave-uniform), written as inline assembly.  The compiler's own wait
// counting knows nothing of it, so its waits only become stricter (one more
// load in flight than it counts); the builtin form instead made it wait for
// every load in flight before each LDS read of the walk while a copy might
// still be pending, which serialized the tile pipeline.  The LDS is read
// only after an explicit wait for all of the wave's loads.
__device__ __forceinline__ void dma_dword(const uint8_t* g, uint8_t* lds) {
  typedef __attribute__((address_space(3))) uint8_t lds_u8_t;
  const uint32_t base = static_cast<uint32_t>(reinterpret_cast<size_t>((lds_u8_t*)(lds)));
  asm volatile("global_load_lds_dword %0, off" ::"v"(g), "{m0}"(base) : "memory");
}

// Orders one wave's LDS write before its later LDS read.  LDS instructions of
// a wave execute in order, so no instruction is needed; the fences only keep
// the compiler from moving the accesses across this point.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Per-wave online-softmax state and the work on one tile of TT tokens (16,
// or 32: whole rows of a 32-token block).  A tile row is NSEG 16-byte
// segments, so one load covers R = 64 / NSEG rows; after the reduce-scatter
// SH = 64 / TT adjacent lanes hold the same token.
template <DT QDT, DT CDT, int D, int TT = kTileTokens>
struct ValuWave {
  static constexpr int E = Elem<CDT>::bytes;
  static constexpr int NSEG = TT * E / 16;
  static constexpr int R = 64 / NSEG;
  static constexpr int TPS = 16 / E;
  static constexpr int SH = 64 / TT;
  static constexpr int kLogSH = SH == 4 ? 2 : 1;
  static_assert(TT == 16 || (TT == 32 && E <= 2), "tile width");
  // loads per lane: R rows each; when D is not a multiple of R, the lanes
  // of the last load past row D - 1 read row D - 1 again (their q is 0 and
  // their results are never written)
  static constexpr int NL = (D + R - 1) / R;
  static constexpr bool kRagged = D % R != 0;

  // q as loaded, converted where it is used (so that nothing waits for it
  // before the walk's first tiles are requested); the score scale is applied
  // per token.  q_last_ok: whether the lane's last row is its own (a lane
  // past row D - 1 reads row D - 1 and uses 0).
  typename Elem<QDT>::storage qraw[NL];
  float acc[NL];
  float m, l, qk_scale;
  int r, seg, L;
  bool q_last_ok;

  // Scores of one tile (tokens tb .. tb + TT - 1): the online-softmax update
  // of (m, l), the probabilities to p_lds[buf]; returns the factor that
  // rescales the earlier weighted sum.  Tokens at L and past it never count;
  // MASKED: bit t of okmask says whether tile token t comes from a valid
  // block (block size 8, a 16-token tile over two blocks); RANGE: only the
  // tokens in [lo, hi) count (hi <= L; 32-token tiles over two blocks).
  template <bool MASKED = false, bool RANGE = false>
  __device__ __forceinline__ float scores(const uint4 (&kr)[NL], int tb, float (*p_lds)[TT],
                                          int buf, uint32_t okmask = 0xFFFFu, int lo = 0,
                                          int hi = 0) {
    // q . K for the lane's TPS tokens, partial over its NL rows
    float part_[TPS];
#pragma unroll
    for (int t = 0; t < TPS; ++t) part_[t] = 0.f;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      // the empty asm keeps the conversion here, per tile: hoisted before
      // the walk it would wait for q before the first tiles are requested
      auto qr = qraw[i];
      asm volatile("" : "+v"(qr));
      const float qf = (i < NL - 1 || q_last_ok) ? load_f32<QDT>(&qr) : 0.f;
      float kf[TPS];
      segment_to_f32<CDT>(kr[i], kf);
#pragma unroll
      for (int t = 0; t < TPS; ++t) part_[t] = fmaf(qf, kf[t], part_[t]);
    }
    reduce_scatter<R / 2, TPS>(part_, r);
    float x = part_[0];
    if constexpr (SH == 4) x += xor_lane<2>(x);
    x += xor_lane<1>(x);
    x *= qk_scale;

    const int tok = tb + seg * TPS + (r >> kLogSH);
    if constexpr (RANGE) {
      if (tok >= hi || tok < lo) x = -INFINITY;
    } else {
      if (tok >= L) x = -INFINITY;
    }
    if constexpr (MASKED) {
      if (!((okmask >> (seg * TPS + (r >> kLogSH))) & 1u)) x = -INFINITY;
    }

    const float m_new = fmaxf(m, seg_max<SH, R>(x));
    // a segment can have seen no valid token yet (m_new = -inf): use 0 as the
    // reference then, so that exp2(-inf - ref) = 0 instead of NaN
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_ref);
    const float pr = fast_exp2(x - m_ref);
    l = fmaf(l, alpha, pr);
    m = m_new;

    if ((r & (SH - 1)) == 0) p_lds[buf][seg * TPS + (r >> kLogSH)] = pr;
    return alpha;
  }

  // The weighted sum over one tile's V rows with the probabilities that
  // scores() left in p_lds[buf], after rescaling the earlier sum by alpha.
  template <bool MASKED = false, bool RANGE = false>
  __device__ __forceinline__ void accumulate(const uint4 (&vr)[NL], float alpha, int tb,
                                             float (*p_lds)[TT], int buf,
                                             uint32_t okmask = 0xFFFFu, int lo = 0, int hi = 0) {
    wave_lds_sync();
    float pv[TPS];
#pragma unroll
    for (int t = 0; t < TPS; ++t) pv[t] = p_lds[buf][seg * TPS + t];

    const bool partial = MASKED || (RANGE ? (tb + TT > hi || lo > tb) : tb + TT > L);
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      float vf[TPS];
      segment_to_f32<CDT>(vr[i], vf);
      float a = acc[i] * alpha;
#pragma unroll
      for (int t = 0; t < TPS; ++t) {
        // a masked token has p = 0, but its V may hold NaN: zero it too
        bool off;
        if constexpr (RANGE) off = tb + seg * TPS + t >= hi || tb + seg * TPS + t < lo;
        else off = tb + seg * TPS + t >= L;
        if constexpr (MASKED) off = off || !((okmask >> (seg * TPS + t)) & 1u);
        const float vv = (partial && off) ? 0.f : vf[t];
        a = fmaf(pv[t], vv, a);
      }
      acc[i] = a;
    }
  }

  template <bool MASKED = false>
  __device__ __forceinline__ void block(const uint4 (&kr)[NL], const uint4 (&vr)[NL], int tb,
                                        float (*p_lds)[TT], int buf, uint32_t okmask = 0xFFFFu) {
    const float alpha = scores<MASKED>(kr, tb, p_lds, buf, okmask);
    accumulate<MASKED>(vr, alpha, tb, p_lds, buf, okmask);
  }
};

// NL 16-byte segments of a lane, STRIDE bytes apart (64 * BLOCK_SIZE: the
// R rows of one load instruction times the row length); the last one LAST
// bytes further (0, or the step back to row D - 1 of a lane past it).  Nontemporal when a
// tile is whole rows (BLOCK_SIZE <= 16); at BLOCK_SIZE 32 a tile is half of
// each row and the other half is read right after it, so the lines are kept
// in cache (nontemporal loads there cost a second fetch: 2x slower).
template <int NL, int STRIDE, bool NT = true>
__device__ __forceinline__ void load_tile(const uint8_t* kp, const uint8_t* vp, uint4 (&k)[NL],
                                          uint4 (&v)[NL], int last) {
  auto ld = [](const uint8_t* a) {
    if constexpr (NT) return load_nt16(a);
    else return *reinterpret_cast<const uint4*>(a);
  };
#pragma unroll
  for (int i = 0; i < NL; ++i) k[i] = ld(kp + i * STRIDE + (i == NL - 1 ? last : 0));
#pragma unroll
  for (int i = 0; i < NL; ++i) v[i] = ld(vp + i * STRIDE + (i == NL - 1 ? last : 0));
}

// FP8 at BLOCK_SIZE 8: a lane's 16 tokens are two 8-byte rows of two blocks.
template <int NL, int STRIDE>
__device__ __forceinline__ void load_tile_split(const uint8_t* k0, const uint8_t* k1,
                                                const uint8_t* v0, const uint8_t* v1,
                                                uint4 (&k)[NL], uint4 (&v)[NL], int last) {
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int o = i * STRIDE + (i == NL - 1 ? last : 0);
    const u32x2_t a = load_nt8(k0 + o), b = load_nt8(k1 + o);
    k[i] = uint4{a[0], a[1], b[0], b[1]};
  }
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int o = i * STRIDE + (i == NL - 1 ? last : 0);
    const u32x2_t a = load_nt8(v0 + o), b = load_nt8(v1 + o);
    v[i] = uint4{a[0], a[1], b[0], b[1]};
  }
}

// Stores of a tile, mirroring load_tile / load_tile_split (decode with
// append: the tile holding the new token goes back whole, so every cache line
// of it is written completely).  last_ok: whether the lane's last segment is
// its own row (a lane past row D - 1 stores nothing there).
template <int NL, int STRIDE>
__device__ __forceinline__ void store_tile(uint8_t* kp, uint8_t* vp, const uint4 (&k)[NL],
                                           const uint4 (&v)[NL], bool last_ok) {
#pragma unroll
  for (int i = 0; i < NL; ++i)
    if (i < NL - 1 || last_ok) *reinterpret_cast<uint4*>(kp + i * STRIDE) = k[i];
#pragma unroll
  for (int i = 0; i < NL; ++i)
    if (i < NL - 1 || last_ok) *reinterpret_cast<uint4*>(vp + i * STRIDE) = v[i];
}
// FP8 at BLOCK_SIZE 8: writes back the 8-byte half from block h (0: k0/v0,
// 1: k1/v1) of each lane's segment.
template <int NL, int STRIDE>
__device__ __forceinline__ void store_tile_half(uint8_t* kp, uint8_t* vp, const uint4 (&k)[NL],
                                                const uint4 (&v)[NL], int h, bool last_ok) {
#pragma unroll
  for (int i = 0; i < NL; ++i)
    if (i < NL - 1 || last_ok)
      *reinterpret_cast<u32x2_t*>(kp + i * STRIDE) =
          h ? u32x2_t{k[i].z, k[i].w} : u32x2_t{k[i].x, k[i].y};
#pragma unroll
  for (int i = 0; i < NL; ++i)
    if (i < NL - 1 || last_ok)
      *reinterpret_cast<u32x2_t*>(vp + i * STRIDE) =
          h ? u32x2_t{v[i].z, v[i].w} : u32x2_t{v[i].x, v[i].y};
}

// Replaces element e (E bytes) of a 16-byte segment.
template <int E>
__device__ __forceinline__ void put_element(uint4& v, int e, uint32_t bits) {
  const int dw = (e * E) >> 2;
  const int sh = ((e * E) & 3) * 8;
  const uint32_t mask = E == 4 ? 0xffffffffu : ((1u << (8 * E)) - 1u) << sh;
  const uint32_t b = (bits << sh) & mask;
  v.x = dw == 0 ? (v.x & ~mask) | b : v.x;
  v.y = dw == 1 ? (v.y & ~mask) | b : v.y;
  v.z = dw == 2 ? (v.z & ~mask) | b : v.z;
  v.w = dw == 3 ? (v.w & ~mask) | b : v.w;
}

template <DT QDT, DT CDT, int D, int BS>
__global__ __launch_bounds__(64 * kWaves) void decode_valu_kernel(DecodePtrs ptr,
                                                                      DecodeParams p) {
  // 16-bit and E4M3 caches walk 32-token tiles: at BLOCK_SIZE 32 a block
  // (whole 64- or 32-byte rows), at 16 two consecutive blocks; float32 caches
  // and BLOCK_SIZE 8 walk 16-token tiles
  constexpr int TT = (BS == 32 || BS == 16) && Elem<CDT>::bytes <= 2 ? 32 : kTileTokens;
  constexpr bool kWhole32 = TT == 32;
  using W = ValuWave<QDT, CDT, D, TT>;
  constexpr int E = W::E, R = W::R, NL = W::NL, TPS = W::TPS, NSEG = W::NSEG;
  // one (block, kv head) tile of the cache: head_size rows of BS tokens
  constexpr size_t kTileBytes = size_t(D) * BS * E;
  constexpr int kStride = R * BS * E;              // bytes between a lane's loads
  constexpr int kTilesPerBlock = BS >= kTileTokens ? BS / kTileTokens : 1;
  constexpr bool kTwoBlocks = BS < kTileTokens;    // a 16-token tile spans two blocks
  constexpr bool kSplit = kTwoBlocks && TPS > BS;  // FP8: a lane's segment spans both
  static_assert(BS == 8 || BS == 16 || BS == 32, "block size");
  using QS = typename Elem<QDT>::storage;

  __shared__ float p_lds[kWaves][2][TT];     // probabilities, per wave
  __shared__ float c_acc[kWaves][D];         // per-wave partial results
  __shared__ float c_m[kWaves], c_l[kWaves];
  __shared__ int item[3];                    // the item's sequence, length, partition (plain)
  // the new token's key and value rows, per wave (decode with append)
  constexpr int kNewPieces = (D * Elem<QDT>::bytes + 255) / 256;
  __shared__ __attribute__((aligned(16))) uint8_t new_lds[kWaves][2][kNewPieces * 256];

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  W w;
  w.r = lane % R;
  w.seg = lane / R;
  // Work item order: head fastest, then sequence, then partition, with
  // work-groups taken in id order.  The hardware deals ids round-robin to the
  // 8 XCDs, so the heads of one block (a contiguous run of tiles) are read
  // through all eight XCDs at once; keeping them on one XCD measured 20%
  // slower on the LLaMA-7B-shaped batch.
  const int unit = blockIdx.x;
  const int h = unit % p.H;
  int s, part, l_raw, first = 0;
  if (p.group_starts == nullptr) {
    // longest-first order; the ids past the last item come last and exit
    if (wid == 0) {                                // one search per work-group
      int len = 0, pt = 0;
      const int s0 = longest_first_sequence(unit / p.H, p.np_run, p.bpp, ptr.context_lens, p.S,
                                            p.cap, pt, len);
      if (lane == 0) {
        item[0] = s0;
        item[1] = len;
        item[2] = pt;
      }
    }
    __syncthreads();
    s = __builtin_amdgcn_readfirstlane(item[0]);
    if (s < 0) return;                             // past the last item: the group leaves
    l_raw = __builtin_amdgcn_readfirstlane(item[1]);
    part = __builtin_amdgcn_readfirstlane(item[2]);
  } else {
    // suffix pass of a shared-prefix batch (BLOCK_SIZE 16: tiles are
    // blocks): index order, blocks after the group's prefix, results from
    // workspace slot slot0 on
    part = unit / (p.H * p.S);
    s = (unit / p.H) % p.S;
    first = group_prefix_blocks(s, p);
    l_raw = ptr.context_lens[s];
  }

  const int nb = tiles_of(l_raw, p.cap);             // 16-token tiles
  w.L = tokens_of(l_raw, p.cap);
  const int nbs = nb > first ? nb - first : 0;      // tiles this pass covers
  const int nparts = nbs == 0 ? 1 : (nbs + p.bpp - 1) / p.bpp;
  if (part >= nparts) {                             // suffix pass only: empty partial
    if (threadIdx.x == 0) {                         // (its weighted sum is never read)
      const size_t base = (size_t(s) * p.H + h) * p.np + p.slot0 + part;
      p.ws_m[base] = -INFINITY;
      p.ws_l[base] = 0.f;
    }
    return;
  }

  const int kvh = h / p.g;
  const QS* q = reinterpret_cast<const QS*>(ptr.query) + size_t(s) * p.q_stride + size_t(h) * D;
  // row of the lane's last load, and whether it is the lane's own
  const int row_last = (NL - 1) * R + w.r;
  const bool last_ok = !W::kRagged || row_last < D;
  auto load_q = [&]() {
#pragma unroll
    for (int i = 0; i < NL; ++i) w.qraw[i] = q[i < NL - 1 || last_ok ? i * R + w.r : D - 1];
  };
  // (block size 16 loads q after its first tiles are requested)
  w.q_last_ok = last_ok;
  w.qk_scale = p.qk_scale;

  // The sequence's tiles are split into nparts nearly equal runs (sizes
  // differ by at most one tile), so no partition is a small remainder; the
  // work-group's run is split the same way among its waves.
  const int pj0 = first + (part * nbs) / nparts;
  const int pj1 = first + ((part + 1) * nbs) / nparts;
  const int j0 = pj0 + (wid * (pj1 - pj0)) / kWaves;
  const int j1 = pj0 + ((wid + 1) * (pj1 - pj0)) / kWaves;
  const int32_t* bt = ptr.block_tables + size_t(s) * p.MB;
  // lane's row r and segment: for BLOCK_SIZE >= 16 at 16-byte segment seg of
  // the tile's row (plus 16 tokens per earlier tile of the same block); for
  // BLOCK_SIZE 8 in block 2t + half, at the segment's place in the 8-token row
  const int half = kTwoBlocks && !kSplit ? (w.seg * TPS) / BS : 0;
  constexpr int kSpr = BS * E / 16 > 0 ? BS * E / 16 : 1;   // 16-byte segments per block row
  const size_t lane_off = size_t(kvh) * kTileBytes + size_t(w.r) * (BS * E) +
                          (kTwoBlocks ? ((w.seg * TPS) % BS) * E : (w.seg % kSpr) * 16);
  const size_t block_stride = size_t(p.Hk) * kTileBytes;
  const uint8_t* kbase = ptr.kcache + lane_off;
  const uint8_t* vbase = ptr.vcache + lane_off;
  const int last = last_ok ? 0 : (D - 1 - row_last) * BS * E;   // bytes, <= 0
  float (*my_lds)[TT] = p_lds[wid];
  const int nblk = (w.L + BS - 1) / BS;              // blocks holding the tokens

  // Decode with append: the wave whose tiles include logical position L - 1
  // puts the new token into its registers before computing that tile (every
  // query head of the KV head does), and the first query head of the KV head
  // stores the tile back.  Tokens are tile t_new's element o_new.
  const bool appending = p.knew != nullptr && l_raw >= 1 && l_raw <= p.cap;
  const int t_new = appending ? (l_raw - 1) / TT : -1;
  const int o_new = (l_raw - 1) & (TT - 1);
  const bool stores_new = h % p.g == 0;
  // The new token's key and value rows (this KV head) are copied into the
  // wave's LDS by the direct global->LDS load, requested behind the walk's
  // first tiles, so that they have long arrived when the last tile (the one
  // that takes the token) is reached.  Loaded there instead, they cost the
  // wave one more memory round trip at the end of its walk, which the whole
  // work-group waited for.  Every wave requests them (the q row stands in
  // when the call does not append), so that its load counts are the same on
  // every path.
  constexpr int ES = Elem<QDT>::bytes;
  const uint8_t* krow = appending ? p.knew + (size_t(s) * p.kn_stride + size_t(kvh) * D) * ES
                                  : reinterpret_cast<const uint8_t*>(q);
  const uint8_t* vrow = appending ? p.vnew + (size_t(s) * p.vn_stride + size_t(kvh) * D) * ES
                                  : reinterpret_cast<const uint8_t*>(q);
  auto load_new = [&]() {
#pragma unroll
    for (int c = 0; c < kNewPieces; ++c) {
      // 4 bytes per lane; lanes past the row re-read its first bytes
      const int o = c * 256 + lane * 4 < D * ES ? c * 256 + lane * 4 : 0;
      dma_dword(krow + o, new_lds[wid][0] + c * 256);
      dma_dword(vrow + o, new_lds[wid][1] + c * 256);
    }
  };
  auto put_new = [&](uint4 (&k)[NL], uint4 (&v)[NL]) {
    // the rows have landed (the tile taking the token is the wave's last:
    // no later load is in flight)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (w.seg == o_new / TPS) {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int d = i < NL - 1 || last_ok ? i * R + w.r : D - 1;
        put_element<E>(k[i], o_new % TPS, new_token_bits<QDT, CDT>(new_lds[wid][0], d, p.enc_k));
        put_element<E>(v[i], o_new % TPS, new_token_bits<QDT, CDT>(new_lds[wid][1], d, p.enc_v));
      }
    }
  };
  // the same for a K or a V tile alone (rows: the token's row in LDS, landed)
  auto put_rows = [&](uint4 (&t)[NL], const uint8_t* rows, float enc) {
    if (w.seg == o_new / TPS) {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int d = i < NL - 1 || last_ok ? i * R + w.r : D - 1;
        put_element<E>(t[i], o_new % TPS, new_token_bits<QDT, CDT>(rows, d, enc));
      }
    }
  };

  if constexpr ((kTilesPerBlock == 2 && !kWhole32) || kTwoBlocks) {
    load_new();
    load_q();
  }

  w.m = -INFINITY;
  w.l = 0.f;
#pragma unroll
  for (int i = 0; i < NL; ++i) w.acc[i] = 0.f;

  // Walk the wave's tiles 64 at a time: one vector load fetches the table
  // ids, each tile reads its id(s) with readlane.  Tile j+1 is in flight
  // while tile j is computed (two register sets, used alternately).  Loads
  // are unconditional so that the wait counts stay exact: an id outside the
  // pool reads block 0 instead and its tokens are skipped; the prefetch after
  // the last tile re-reads that tile (an L2 hit).
  int buf = 0;
  auto valid = [&](int phys) { return static_cast<unsigned>(phys) < static_cast<unsigned>(p.NB); };
  auto at = [&](const uint8_t* base, int phys) {
    return base + size_t(valid(phys) ? phys : 0) * block_stride;
  };
  // the lane's bytes of (valid) block phys in a cache, for the stores of the
  // append (the same address as at(), writable)
  auto wat = [&](const uint8_t* cache, int phys) {
    return const_cast<uint8_t*>(cache) + size_t(phys) * block_stride + lane_off;
  };
  if constexpr (kWhole32) {
    // 32-token tiles, read as whole block rows: at BLOCK_SIZE 32 tile t is
    // block t; at 16 it is blocks fb + 2t and fb + 2t + 1 (fb = first, the
    // pass's first block), the lanes of a row's first two (E4M3: first)
    // 16-byte segments reading the first block and the others the second, so
    // that each load moves 512 contiguous bytes of each.  The partition's and
    // the waves' runs are split in tiles.  K and V of a tile are separate
    // steps of the pipeline: tile t + 1's K is requested once tile t's scores
    // are computed, its V once tile t's weighted sum is, so one of them is in
    // flight while the other is computed, within the registers of one tile.
    constexpr bool kPair = BS == 16;
    const int fb = kPair ? first : 0;
    const int ntl = nblk <= fb ? 0 : kPair ? (nblk - fb + 1) / 2 : nblk;
    const int pb0 = (part * ntl) / nparts;
    const int pb1 = ((part + 1) * ntl) / nparts;
    const int b0 = pb0 + (wid * (pb1 - pb0)) / kWaves;
    const int b1 = pb0 + ((wid + 1) * (pb1 - pb0)) / kWaves;
    const int hb = kPair ? w.seg / kSpr : 0;             // the lane's block of the pair
    auto ld = [&](const uint8_t* a, uint4 (&t)[NL]) {
#pragma unroll
      for (int i = 0; i < NL; ++i) t[i] = load_nt16(a + i * kStride + (i == NL - 1 ? last : 0));
    };
    auto st = [&](uint8_t* a, const uint4 (&t)[NL]) {
#pragma unroll
      for (int i = 0; i < NL; ++i)
        if (i < NL - 1 || last_ok) *reinterpret_cast<uint4*>(a + i * kStride) = t[i];
    };
    // first block of tile t, and whether its pair has a second block
    auto blk = [&](int t) { return kPair ? fb + 2 * t : t; };
    auto has_b = [&](int t) { return kPair && blk(t) + 1 < nblk; };
    // tiles c0 .. c0 + cnt - 1 (1 <= cnt <= 64); with_q: load q there
    auto walk_chunk = [&](int c0, int cnt, bool with_q) {
      const int lt = c0 + (lane < cnt ? lane : cnt - 1);
      const int my_a = bt[blk(lt)];
      const int my_b = has_b(lt) ? bt[blk(lt) + 1] : -1;
      const int id0a = scalar_ptr(bt)[blk(c0)];
      const int id0b = has_b(c0) ? scalar_ptr(bt)[blk(c0) + 1] : -1;
      // the lane's block of tile t (ids a, b); past the sequence's last
      // block the second half re-reads the first (its tokens do not count)
      auto lane_id = [&](int t, int a, int b) { return hb && has_b(t) ? b : a; };
      auto tile_at = [&](const uint8_t* base, int t, int a, int b) {
        return at(base, lane_id(t, a, b));
      };
      // the tokens of tile t that count, [lo, hi): a block whose entry lies
      // outside the pool contributes none (its lanes read block 0)
      auto range = [&](int t, int a, int b, int& lo, int& hi) {
        lo = blk(t) * BS;
        hi = w.L;
        if constexpr (kPair) {
          const int mid = lo + BS;                     // the second block's first token
          if (!valid(a)) lo = mid;
          if (has_b(t) && !valid(b)) hi = mid < hi ? mid : hi;
        } else {
          if (!valid(a)) hi = lo;
        }
      };
      uint4 k[NL], v[NL];
      int ia = id0a, ib = id0b;
      int id = lane_id(c0, ia, ib);
      ld(tile_at(kbase, c0, ia, ib), k);
      ld(tile_at(vbase, c0, ia, ib), v);
      if (with_q) {                                    // behind the first tile, not before it
        load_new();
        load_q();
      }
      for (int jj = 0; jj < cnt; ++jj) {
        const bool more = jj + 1 < cnt;
        const int na = more ? __builtin_amdgcn_readlane(my_a, jj + 1) : 0;
        const int nbb = more && kPair ? __builtin_amdgcn_readlane(my_b, jj + 1) : -1;
        const int nid = lane_id(c0 + jj + 1, na, nbb);
        const int tb = blk(c0 + jj) * BS;
        int lo, hi;
        range(c0 + jj, ia, ib, lo, hi);
        const bool ok = hi > lo;
        // (the call appends only with fb = 0: tile t_new holds position L - 1)
        const bool is_new = c0 + jj == t_new;
        // the lanes of the block that holds the new token store it back
        const bool st_new = stores_new && (!kPair || hb == o_new / BS) && valid(id);
        float alpha = 1.f;
        if (ok) {
          if (is_new) {
            // the new rows have landed (this tile's V may still be in flight)
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            put_rows(k, new_lds[wid][0], p.enc_k);
            if (st_new) st(wat(ptr.kcache, id), k);
          }
          alpha = w.template scores<false, true>(k, tb, my_lds, buf, 0u, lo, hi);
        } else {
#pragma unroll
          for (int i = 0; i < NL; ++i) asm volatile("" ::"v"(k[i].x));
        }
        if (more) ld(tile_at(kbase, c0 + jj + 1, na, nbb), k);
        if (ok) {
          if (is_new) {
            put_rows(v, new_lds[wid][1], p.enc_v);
            if (st_new) st(wat(ptr.vcache, id), v);
          }
          w.template accumulate<false, true>(v, alpha, tb, my_lds, buf, 0u, lo, hi);
          buf ^= 1;
        } else {
#pragma unroll
          for (int i = 0; i < NL; ++i) asm volatile("" ::"v"(v[i].x));
        }
        if (more) ld(tile_at(vbase, c0 + jj + 1, na, nbb), v);
        id = nid;
        ia = na;
        ib = nbb;
      }
      asm volatile("" ::"v"(my_a), "v"(my_b));          // (the table rows too, when unused)
    };
    if (b1 - b0 <= 64) {
      if (b1 > b0) walk_chunk(b0, b1 - b0, true);
    } else {
      load_new();
      load_q();
      for (int c0 = b0; c0 < b1; c0 += 64) walk_chunk(c0, (b1 - c0) < 64 ? (b1 - c0) : 64, false);
    }
  } else if constexpr (kTilesPerBlock == 2) {
    // BLOCK_SIZE 32: tiles 2b and 2b + 1 are the two 16-token halves of each
    // row of block b.  Both halves are loaded back to back and then computed,
    // so the second half's loads find the lines the first half's brought in
    // (cache-allocating loads; 6% faster than alternating halves with the
    // next tile in flight, and nontemporal loads there cost a second fetch).
    for (int c0 = j0; c0 < j1; c0 += 64) {
      const int cnt = (j1 - c0) < 64 ? (j1 - c0) : 64;
      const int my_id = lane < cnt ? bt[(c0 + lane) / 2] : 0;
      auto id_at = [&](int jj) { return __builtin_amdgcn_readlane(my_id, jj); };
      uint4 ka[NL], va[NL], kb[NL], vb[NL];
      constexpr int kHalf = kTileTokens * E;          // bytes from a row's first half to its second
      auto single = [&](int jj) {                      // one half-block tile
        const int id = id_at(jj);
        const int off = ((c0 + jj) & 1) * kHalf;
        load_tile<NL, kStride, false>(at(kbase, id) + off, at(vbase, id) + off, ka, va, last);
        if (valid(id)) {
          if (c0 + jj == t_new) {
            put_new(ka, va);
            if (stores_new) store_tile<NL, kStride>(wat(ptr.kcache, id) + off,
                                                    wat(ptr.vcache, id) + off, ka, va, last_ok);
          }
          w.block(ka, va, (c0 + jj) * kTileTokens, my_lds, buf);
          buf ^= 1;
        }
      };
      int jj = 0;
      if constexpr (NL > 8) {
        // head sizes of 192 and more: four tile register sets would not fit,
        // so the halves are walked one at a time
        for (; jj < cnt; ++jj) single(jj);
      }
      if ((c0 & 1) != 0 && jj < cnt) single(jj++);     // the walk starts at a second half
      for (; jj + 1 < cnt; jj += 2) {
        const int id = id_at(jj);
        load_tile<NL, kStride, false>(at(kbase, id), at(vbase, id), ka, va, last);
        load_tile<NL, kStride, false>(at(kbase, id) + kHalf, at(vbase, id) + kHalf, kb, vb, last);
        if (valid(id)) {
          if (c0 + jj == t_new || c0 + jj + 1 == t_new) {
            if (c0 + jj == t_new) put_new(ka, va);
            else put_new(kb, vb);
            if (stores_new) {                          // both halves: whole rows
              store_tile<NL, kStride>(wat(ptr.kcache, id), wat(ptr.vcache, id), ka, va, last_ok);
              store_tile<NL, kStride>(wat(ptr.kcache, id) + kHalf, wat(ptr.vcache, id) + kHalf,
                                      kb, vb, last_ok);
            }
          }
          w.block(ka, va, (c0 + jj) * kTileTokens, my_lds, buf);
          buf ^= 1;
          w.block(kb, vb, (c0 + jj + 1) * kTileTokens, my_lds, buf);
          buf ^= 1;
        }
      }
      if (jj < cnt) single(jj);                        // the walk ends at a first half
    }
  } else if constexpr (!kTwoBlocks) {
    // tile t is block t (BLOCK_SIZE 16)
    auto append16 = [&](int id, uint4 (&k)[NL], uint4 (&v)[NL]) {
      put_new(k, v);
      if (stores_new) store_tile<NL, kStride>(wat(ptr.kcache, id), wat(ptr.vcache, id), k, v, last_ok);
    };
    // tiles c0 .. c0 + cnt - 1 (1 <= cnt <= 64); with_q: load q there
    auto walk_chunk = [&](int c0, int cnt, bool with_q) {
      // (every lane loads, lanes past cnt the last entry: no branch, so no
      // wait at a join before the first tiles are requested)
      const int my_id = bt[c0 + (lane < cnt ? lane : cnt - 1)];
      // the first two ids through the scalar cache (they start the walk);
      // the rest from the vector load, long arrived when they are needed
      const int id0 = scalar_ptr(bt)[c0];
      const int id1 = scalar_ptr(bt)[c0 + (cnt > 1 ? 1 : 0)];
      auto id_at = [&](int jj) {
        return jj == 0 ? id0 : jj == 1 ? id1 : __builtin_amdgcn_readlane(my_id, jj);
      };
      uint4 ka[NL], va[NL], kb[NL], vb[NL];
      auto run = [&](int id, int jj, uint4 (&k)[NL], uint4 (&v)[NL]) {
        if (valid(id)) {
          if (c0 + jj == t_new) append16(id, k, v);
          w.block(k, v, (c0 + jj) * kTileTokens, my_lds, buf);
          buf ^= 1;
        } else {
          // not computed, but consumed all the same (so that no load is left
          // in flight, as the pair loop below requires)
#pragma unroll
          for (int i = 0; i < NL; ++i) asm volatile("" ::"v"(k[i].x), "v"(v[i].x));
        }
      };
      int ia = id_at(0);
      load_tile<NL, kStride>(at(kbase, ia), at(vbase, ia), ka, va, last);
      if (with_q) {                                    // behind the first tiles, not before them
        load_new();
        load_q();
      }
      int jj = 0;
      // pairs while a third tile follows, then the last one or two: every
      // tile loaded is used, so no load is left in flight at the chunk's end
      // (one would make the next chunk's first loads wait for all before it)
      for (; jj + 2 < cnt; jj += 2) {
        const int ib = id_at(jj + 1);
        load_tile<NL, kStride>(at(kbase, ib), at(vbase, ib), kb, vb, last);
        run(ia, jj, ka, va);
        const int ia2 = id_at(jj + 2);
        load_tile<NL, kStride>(at(kbase, ia2), at(vbase, ia2), ka, va, last);
        run(ib, jj + 1, kb, vb);
        ia = ia2;
      }
      if (jj + 1 < cnt) {
        const int ib = id_at(jj + 1);
        load_tile<NL, kStride>(at(kbase, ib), at(vbase, ib), kb, vb, last);
        run(ia, jj, ka, va);
        run(ib, jj + 1, kb, vb);
      } else {
        run(ia, jj, ka, va);
      }
      asm volatile("" ::"v"(my_id));                   // (the table row too, when unused)
    };
    // a wave's run is nearly always one chunk: walked outside any loop, so
    // that no loop-carried state makes the first tiles wait for q
    if (j1 - j0 <= 64) {
      if (j1 > j0) walk_chunk(j0, j1 - j0, true);
    } else {
      load_new();
      load_q();
      for (int c0 = j0; c0 < j1; c0 += 64) walk_chunk(c0, (j1 - c0) < 64 ? (j1 - c0) : 64, false);
    }
  } else {
    // BLOCK_SIZE 8: tile t is blocks 2t and 2t + 1 (the second may lie past
    // the sequence's last block); each half's tokens count only when its
    // block id is valid
    for (int c0 = j0; c0 < j1; c0 += 64) {
      const int cnt = (j1 - c0) < 64 ? (j1 - c0) : 64;
      const int b0 = 2 * (c0 + lane);
      const int my_id0 = lane < cnt ? bt[b0] : 0;
      const int my_id1 = lane < cnt && b0 + 1 < nblk ? bt[b0 + 1] : -1;
      auto tile = [&](int jj, uint4 (&k)[NL], uint4 (&v)[NL]) {
        const int i0 = __builtin_amdgcn_readlane(my_id0, jj);
        const int i1 = __builtin_amdgcn_readlane(my_id1, jj);
        if constexpr (kSplit) {
          load_tile_split<NL, kStride>(at(kbase, i0), at(kbase, i1), at(vbase, i0),
                                       at(vbase, i1), k, v, last);
        } else {
          const int mine = half ? i1 : i0;
          load_tile<NL, kStride>(at(kbase, mine), at(vbase, mine), k, v, last);
        }
        return (valid(i0) ? 0x00FFu : 0u) | (valid(i1) ? 0xFF00u : 0u);
      };
      // the new token is in block i0 (tile tokens 0..7) or i1 (8..15); only
      // that block's rows are stored back (a lane's other half may lie in a
      // block past the sequence's end)
      auto append8 = [&](int jj, uint4 (&k)[NL], uint4 (&v)[NL]) {
        put_new(k, v);
        if (!stores_new) return;
        const int nh = o_new / BS;                     // 0: block i0, 1: block i1
        const int id = __builtin_amdgcn_readlane(nh ? my_id1 : my_id0, jj);
        if (!valid(id)) return;
        if constexpr (kSplit) {
          store_tile_half<NL, kStride>(wat(ptr.kcache, id), wat(ptr.vcache, id), k, v, nh, last_ok);
        } else if (half == nh) {
          store_tile<NL, kStride>(wat(ptr.kcache, id), wat(ptr.vcache, id), k, v, last_ok);
        }
      };
      uint4 ka[NL], va[NL], kb[NL], vb[NL];
      uint32_t oka = tile(0, ka, va);
      int jj = 0;
      for (; jj + 1 < cnt; jj += 2) {
        const uint32_t okb = tile(jj + 1, kb, vb);
        if (oka) {
          if (c0 + jj == t_new) append8(jj, ka, va);
          w.template block<true>(ka, va, (c0 + jj) * kTileTokens, my_lds, buf, oka);
          buf ^= 1;
        }
        const uint32_t oka2 = tile(jj + 2 < cnt ? jj + 2 : jj + 1, ka, va);
        if (okb) {
          if (c0 + jj + 1 == t_new) append8(jj + 1, kb, vb);
          w.template block<true>(kb, vb, (c0 + jj + 1) * kTileTokens, my_lds, buf, okb);
          buf ^= 1;
        }
        oka = oka2;
      }
      if (jj < cnt && oka) {
        if (c0 + jj == t_new) append8(jj, ka, va);
        w.template block<true>(ka, va, (c0 + jj) * kTileTokens, my_lds, buf, oka);
        buf ^= 1;
      }
    }
  }
  const int r = w.r, seg = w.seg;
  float m = w.m, l = w.l;
  float* acc = w.acc;

  // combine inside the wave: sum of exponentials of a segment, then segments
  l = seg_sum<W::SH, R>(l);
  if constexpr (NSEG > 1) {
#pragma unroll
    for (int mask = R; mask < 64; mask <<= 1) {
      const int src = (lane ^ mask) << 2;
      const float mo = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(m)));
      const float lo = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(l)));
      const float mn = fmaxf(m, mo);
      const float a = (m == -INFINITY) ? 0.f : fast_exp2(m - mn);
      const float b = (mo == -INFINITY) ? 0.f : fast_exp2(mo - mn);
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const float ao = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(acc[i])));
        acc[i] = acc[i] * a + ao * b;
      }
      l = l * a + lo * b;
      m = mn;
    }
  }

  // combine the waves of the work-group through LDS
#pragma unroll
  for (int i = 0; i < NL; ++i)
    if (i % NSEG == seg && (i < NL - 1 || last_ok)) c_acc[wid][i * R + r] = acc[i];
  if (lane == 0) {
    c_m[wid] = m;
    c_l[wid] = l;
  }
  __syncthreads();
  const int tid = threadIdx.x;
  if (tid < D) {
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) M = fmaxf(M, c_m[k]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) {
      const float wk = c_m[k] == -INFINITY ? 0.f : fast_exp2(c_m[k] - M);
      num = fmaf(wk, c_acc[k][tid], num);
      den = fmaf(wk, c_l[k], den);
    }
    if (nparts == 1 && p.group_starts == nullptr) {
      QS* o = reinterpret_cast<QS*>(ptr.out) + size_t(s) * p.o_stride + size_t(h) * D;
      o[tid] = from_f32<QDT>(den > 0.f ? num * (p.v_scale / den) : 0.f);
    } else {
      const size_t base = (size_t(s) * p.H + h) * p.np + p.slot0 + part;
      if (tid == 0) {
        p.ws_m[base] = M;
        p.ws_l[base] = den;
      }
      p.ws_acc[base * D + tid] = num;
    }
  }
}

// Cross-partition merge by log-sum-exp ([TGI] §4.1: the V2 reduction over
// partitions).  WPU waves per (sequence, head) (1, or 4 when a sequence may
// have more than 16 partitions), kMergeWaves per work-group.  Every wave
// reads all partitions' (max, sum), lane k partition k, so the statistics
// arrive in one round trip; the maximum and the weighted sum of sums are wave
// reductions.  The partitions' weighted sums are then split into WPU
// contiguous runs, one per wave, each lane combining its head_size / 64
// elements over up to 16 partitions per round trip (all their loads issued
// before the first is used); with WPU > 1 the waves' sums add up through
// LDS.  A partition of weight 0 (no token, or negligible)
// contributes nothing and its weighted sum is not used (an empty slot's is
// never written).
constexpr int kMergeWaves = 4;
constexpr int kMergeBatch = 16;                    // partitions per round trip

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, xor_lane<1>(v));
  v = fmaxf(v, xor_lane<2>(v));
  v = fmaxf(v, xor_lane<4>(v));
  v = fmaxf(v, xor_lane<8>(v));
  v = fmaxf(v, xor_lane<16>(v));
  return fmaxf(v, xor_lane<32>(v));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += xor_lane<1>(v);
  v += xor_lane<2>(v);
  v += xor_lane<4>(v);
  v += xor_lane<8>(v);
  v += xor_lane<16>(v);
  return v + xor_lane<32>(v);
}

template <DT QDT, int D, int WPU>
__global__ __launch_bounds__(64 * kMergeWaves) void merge_kernel(DecodePtrs ptr, DecodeParams p) {
  static_assert(kMergeWaves % WPU == 0, "waves per unit");
  using QS = typename Elem<QDT>::storage;
  constexpr int EPL = (D + 63) / 64;               // elements per lane (lane + 64 e < D)
  __shared__ float part_num[WPU][WPU > 1 ? EPL * 64 : 1];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int sub = wv % WPU;                        // this wave's run of the unit's partitions
  const int unit = blockIdx.x * (kMergeWaves / WPU) + wv / WPU;
  if (unit >= p.S * p.H) return;                   // whole wave (with WPU > 1: whole work-group)
  const int h = unit % p.H;
  const int s = unit / p.H;
  const size_t base = (size_t(s) * p.H + h) * p.np;
  // the first 64 statistics are requested before the length is known (the
  // addresses do not depend on it; slots past nparts are ignored below)
  const float m_pre = lane < p.np ? p.ws_m[base + lane] : -INFINITY;
  const float l_pre = lane < p.np ? p.ws_l[base + lane] : 0.f;
  int nparts = p.np;                               // shared-prefix batch: every slot is written
  if (p.group_starts == nullptr) {
    const int nb = tiles_of(__builtin_amdgcn_readfirstlane(ptr.context_lens[s]), p.cap);
    nparts = nb == 0 ? 1 : (nb + p.bpp - 1) / p.bpp;
    if (nparts <= 1) return;                       // written by the partition kernel
  }
  auto stat = [&](int k0, float& mk, float& lk) {
    const int k = k0 + lane;
    mk = k < nparts ? (k0 == 0 ? m_pre : p.ws_m[base + k]) : -INFINITY;
    lk = k < nparts ? (k0 == 0 ? l_pre : p.ws_l[base + k]) : 0.f;
  };
  float M = -INFINITY;
  for (int k0 = 0; k0 < nparts; k0 += 64) {        // one pass unless nparts > 64
    float mk, lk;
    stat(k0, mk, lk);
    M = fmaxf(M, wave_max(lk > 0.f ? mk : -INFINITY));
  }
  const int q = (nparts + WPU - 1) / WPU;
  const int k_lo = sub * q;
  const int k_hi = k_lo + q < nparts ? k_lo + q : nparts;
  float den = 0.f, num[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) num[e] = 0.f;
  const float* a = p.ws_acc + base * D + lane;
  for (int k0 = 0; k0 < nparts; k0 += 64) {
    float mk, lk;
    stat(k0, mk, lk);
    const float wk = lk > 0.f ? fast_exp2(mk - M) : 0.f;
    den += wave_sum(wk * lk);
    // this wave's partitions within k0 .. k0 + 63
    const int j_lo = k_lo > k0 ? k_lo - k0 : 0;
    const int j_hi = k_hi - k0 < 64 ? k_hi - k0 : 64;
    for (int j = j_lo; j < j_hi; j += kMergeBatch) {
      float w[kMergeBatch], v[kMergeBatch][EPL];
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        const bool in = j + u < j_hi;                // (uniform)
        w[u] = in ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wk), (j + u) & 63))
                  : 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e)
          v[u][e] = in && lane + 64 * e < D ? a[size_t(k0 + j + u) * D + 64 * e] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u)
#pragma unroll
        for (int e = 0; e < EPL; ++e) num[e] = w[u] != 0.f ? fmaf(w[u], v[u][e], num[e]) : num[e];
    }
  }
  if constexpr (WPU > 1) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) part_num[sub][lane + 64 * e] = num[e];
    __syncthreads();
    if (sub != 0) return;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float t = part_num[0][lane + 64 * e];
#pragma unroll
      for (int w2 = 1; w2 < WPU; ++w2) t += part_num[w2][lane + 64 * e];
      num[e] = t;
    }
  }
  QS* o = reinterpret_cast<QS*>(ptr.out) + size_t(s) * p.o_stride + size_t(h) * D + lane;
#pragma unroll
  for (int e = 0; e < EPL; ++e)
    if (lane + 64 * e < D) o[64 * e] = from_f32<QDT>(den > 0.f ? num[e] * (p.v_scale / den) : 0.f);
}

template <DT Q, DT C, int D, int BS>
hipError_t run_valu(const DecodePtrs& ptr, const DecodeParams& p, hipStream_t stream) {
  const long long units = 1LL * p.np_run * p.S * p.H;
  hipLaunchKernelGGL((decode_valu_kernel<Q, C, D, BS>), dim3(unsigned(units)), dim3(64 * kWaves),
                     0, stream, ptr, p);
  return hipGetLastError();
}

template <DT Q, DT C, int D>
hipError_t by_bs(const DecodePtrs& ptr, const DecodeParams& p, hipStream_t stream) {
  switch (p.lbs) {
    case 3: return run_valu<Q, C, D, 8>(ptr, p, stream);
    case 5: return run_valu<Q, C, D, 32>(ptr, p, stream);
    default: return run_valu<Q, C, D, 16>(ptr, p, stream);
  }
}

template <DT Q, int D>
hipError_t run_merge(const DecodePtrs& ptr, const DecodeParams& p, hipStream_t stream) {
  const long long units = 1LL * p.S * p.H;
  if (p.np > kMergeBatch) {                        // a work-group per unit, its waves split the runs
    hipLaunchKernelGGL((merge_kernel<Q, D, kMergeWaves>), dim3(unsigned(units)),
                       dim3(64 * kMergeWaves), 0, stream, ptr, p);
    return hipGetLastError();
  }
  const unsigned grid = unsigned((units + kMergeWaves - 1) / kMergeWaves);
  hipLaunchKernelGGL((merge_kernel<Q, D, 1>), dim3(grid), dim3(64 * kMergeWaves), 0, stream, ptr, p);
  return hipGetLastError();
}

template <DT Q, DT C>
hipError_t by_d(int D, const DecodePtrs& ptr, const DecodeParams& p, hipStream_t st) {
  switch (D) {
    case 32: return by_bs<Q, C, 32>(ptr, p, st);
    case 64: return by_bs<Q, C, 64>(ptr, p, st);
    case 80: return by_bs<Q, C, 80>(ptr, p, st);
    case 96: return by_bs<Q, C, 96>(ptr, p, st);
    case 112: return by_bs<Q, C, 112>(ptr, p, st);
    case 120: return by_bs<Q, C, 120>(ptr, p, st);
    case 128: return by_bs<Q, C, 128>(ptr, p, st);
    case 192: return by_bs<Q, C, 192>(ptr, p, st);
    case 256: return by_bs<Q, C, 256>(ptr, p, st);
    default: return hipErrorInvalidValue;
  }
}

template <DT Q>
hipError_t merge_by_d(int D, const DecodePtrs& ptr, const DecodeParams& p, hipStream_t st) {
  switch (D) {
    case 32: return run_merge<Q, 32>(ptr, p, st);
    case 64: return run_merge<Q, 64>(ptr, p, st);
    case 80: return run_merge<Q, 80>(ptr, p, st);
    case 96: return run_merge<Q, 96>(ptr, p, st);
    case 112: return run_merge<Q, 112>(ptr, p, st);
    case 120: return run_merge<Q, 120>(ptr, p, st);
    case 128: return run_merge<Q, 128>(ptr, p, st);
    case 192: return run_merge<Q, 192>(ptr, p, st);
    case 256: return run_merge<Q, 256>(ptr, p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_valu(DT q, DT c, int D, const DecodePtrs& ptr, const DecodeParams& p,
                              hipStream_t stream) {
  if (q == DT::F32) return by_d<DT::F32, DT::F32>(D, ptr, p, stream);
  if (q == DT::F16) {
    return c == DT::FP8 ? by_d<DT::F16, DT::FP8>(D, ptr, p, stream)
                        : by_d<DT::F16, DT::F16>(D, ptr, p, stream);
  }
  return c == DT::FP8 ? by_d<DT::BF16, DT::FP8>(D, ptr, p, stream)
                      : by_d<DT::BF16, DT::BF16>(D, ptr, p, stream);
}

hipError_t launch_merge(DT q, int D, const DecodePtrs& ptr, const DecodeParams& p,
                        hipStream_t stream) {
  if (q == DT::F32) return merge_by_d<DT::F32>(D, ptr, p, stream);
  if (q == DT::F16) return merge_by_d<DT::F16>(D, ptr, p, stream);
  return merge_by_d<DT::BF16>(D, ptr, p, stream);
}

}  // namespace pkv
