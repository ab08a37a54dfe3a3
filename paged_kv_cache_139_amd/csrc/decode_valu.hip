// Paged decode attention, one query head per wavefront, on the vector ALUs.
//
// Used when one query head reads each KV head (multi-head attention), and for
// every float32 case.  Work item = (partition, sequence, query head); one
// 64-lane wavefront per work item walks the partition's logical blocks
// through the block table ([L3] "注意力计算的'分页'实现"; [TGI] §4.3) and keeps an
// online softmax; partitions are merged afterwards by merge.hip ([TGI] §4.1,
// V2 partitions + reduction).
//
// Lane layout.  A block's K (or V) tile for one head is head_size rows of 16
// tokens, token fastest ([TGI] §4.2).  Every load instruction moves 1 KiB:
// lane = (row r, segment seg) holds 16 bytes = TPS tokens of one row, where
// E = element bytes, R = 64 / E rows per load, TPS = 16 / E tokens per segment,
// NL = head_size * E / 64 loads per tile.  The query element of each row a lane
// touches is held in a register for the whole partition.
//
// Dot products reduce over rows, i.e. across the R lanes of a segment: a
// reduce-scatter over row-lane bits R/2 .. 4 leaves each lane with one token
// (index r >> 2), then an all-reduce over bits 2 and 1 (DPP quad permutes).
// Each segment keeps its own softmax state (max, sum) so the exponentials of
// a segment never need a cross-segment max; segments are combined once at
// the end of the partition.  Probabilities reach the PV lanes through LDS.
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

template <DT QDT, DT CDT, int D>
__global__ __launch_bounds__(64) void decode_valu_kernel(DecodePtrs ptr, DecodeParams p) {
  constexpr int E = Elem<CDT>::bytes;
  constexpr int R = 64 / E;
  constexpr int TPS = 16 / E;
  constexpr int NL = D * E / 64;
  constexpr size_t kTileBytes = size_t(D) * kBlockSize * E;
  using QS = typename Elem<QDT>::storage;

  __shared__ float p_lds[2][16];

  const int lane = threadIdx.x;
  const int r = lane % R;
  const int seg = lane / R;
  const int unit = xcd_remap(blockIdx.x, gridDim.x);
  const int h = unit % p.H;
  const int s = (unit / p.H) % p.S;
  const int part = unit / (p.H * p.S);

  const int l_raw = ptr.context_lens[s];
  int nb = l_raw > 0 ? (l_raw + kBlockSize - 1) / kBlockSize : 0;
  nb = nb < p.MB ? nb : p.MB;
  const int L = l_raw > 0 ? (l_raw < nb * kBlockSize ? l_raw : nb * kBlockSize) : 0;
  const int nparts = nb == 0 ? 1 : (nb + p.bpp - 1) / p.bpp;
  if (part >= nparts) return;

  const int kvh = h / p.g;
  const QS* q = reinterpret_cast<const QS*>(ptr.query) + (size_t(s) * p.H + h) * D;
  float qv[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) qv[i] = load_f32<QDT>(q + i * R + r) * p.qk_scale;

  const int j0 = part * p.bpp;
  const int j1 = (j0 + p.bpp < nb) ? j0 + p.bpp : nb;
  const int32_t* bt = ptr.block_tables + size_t(s) * p.MB;
  const size_t lane_off = size_t(kvh) * kTileBytes + size_t(r) * (kBlockSize * E) + seg * 16;
  const size_t block_stride = size_t(p.Hk) * kTileBytes;
  const uint8_t* kbase = ptr.kcache + lane_off;
  const uint8_t* vbase = ptr.vcache + lane_off;

  float m = -INFINITY, l = 0.f;
  float acc[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) acc[i] = 0.f;

  int buf = 0;
  for (int j = j0; j < j1; ++j) {
    const int phys = bt[j];
    if (static_cast<unsigned>(phys) >= static_cast<unsigned>(p.NB)) continue;
    const uint8_t* kp = kbase + size_t(phys) * block_stride;
    const uint8_t* vp = vbase + size_t(phys) * block_stride;
    uint4 kr[NL], vr[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) kr[i] = *reinterpret_cast<const uint4*>(kp + i * 1024);
#pragma unroll
    for (int i = 0; i < NL; ++i) vr[i] = *reinterpret_cast<const uint4*>(vp + i * 1024);

    // q . K for the lane's TPS tokens, partial over its NL rows
    float part_[TPS];
#pragma unroll
    for (int t = 0; t < TPS; ++t) part_[t] = 0.f;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      float kf[TPS];
      segment_to_f32<CDT>(kr[i], kf);
#pragma unroll
      for (int t = 0; t < TPS; ++t) part_[t] = fmaf(qv[i], kf[t], part_[t]);
    }
    reduce_scatter<R / 2, TPS>(part_, r);
    float x = part_[0];
    x += xor_lane<2>(x);
    x += xor_lane<1>(x);

    const int tb = j * kBlockSize;
    const int tok = tb + seg * TPS + (r >> 2);
    if (tok >= L) x = -INFINITY;

    const float m_new = fmaxf(m, seg_max<4, R>(x));
    // a segment can have seen no valid token yet (m_new = -inf): use 0 as the
    // reference then, so that exp2(-inf - ref) = 0 instead of NaN
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_ref);
    const float pr = fast_exp2(x - m_ref);
    l = fmaf(l, alpha, pr);
    m = m_new;

    if ((r & 3) == 0) p_lds[buf][seg * TPS + (r >> 2)] = pr;
    __syncthreads();
    float pv[TPS];
#pragma unroll
    for (int t = 0; t < TPS; ++t) pv[t] = p_lds[buf][seg * TPS + t];
    buf ^= 1;

    const bool partial = tb + kBlockSize > L;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      float vf[TPS];
      segment_to_f32<CDT>(vr[i], vf);
      float a = acc[i] * alpha;
#pragma unroll
      for (int t = 0; t < TPS; ++t) {
        // a masked token has p = 0, but its V may hold NaN: zero it too
        const float vv = (partial && tb + seg * TPS + t >= L) ? 0.f : vf[t];
        a = fmaf(pv[t], vv, a);
      }
      acc[i] = a;
    }
  }

  // combine: sum of exponentials inside the segment, then across segments
  l = seg_sum<4, R>(l);
  if constexpr (E > 1) {
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

  if (nparts == 1) {
    QS* o = reinterpret_cast<QS*>(ptr.out) + (size_t(s) * p.H + h) * D;
    const float inv = l > 0.f ? p.v_scale / l : 0.f;
#pragma unroll
    for (int i = 0; i < NL; ++i)
      if (i % E == seg) o[i * R + r] = from_f32<QDT>(acc[i] * inv);
  } else {
    const size_t base = (size_t(s) * p.H + h) * p.np + part;
    if (lane == 0) {
      p.ws_m[base] = m;
      p.ws_l[base] = l;
    }
    float* a = p.ws_acc + base * D;
#pragma unroll
    for (int i = 0; i < NL; ++i)
      if (i % E == seg) a[i * R + r] = acc[i];
  }
}

// Cross-partition merge by log-sum-exp: one thread per head_size element.
template <DT QDT, int D>
__global__ __launch_bounds__(D) void merge_kernel(DecodePtrs ptr, DecodeParams p) {
  using QS = typename Elem<QDT>::storage;
  const int unit = xcd_remap(blockIdx.x, gridDim.x);
  const int h = unit % p.H;
  const int s = unit / p.H;
  const int l_raw = ptr.context_lens[s];
  int nb = l_raw > 0 ? (l_raw + kBlockSize - 1) / kBlockSize : 0;
  nb = nb < p.MB ? nb : p.MB;
  const int nparts = nb == 0 ? 1 : (nb + p.bpp - 1) / p.bpp;
  if (nparts <= 1) return;                 // written by the partition kernel
  const size_t base = (size_t(s) * p.H + h) * p.np;
  float M = -INFINITY;
  for (int k = 0; k < nparts; ++k) M = fmaxf(M, p.ws_m[base + k]);
  float num = 0.f, den = 0.f;
  for (int k = 0; k < nparts; ++k) {
    const float lk = p.ws_l[base + k];
    const float w = lk > 0.f ? fast_exp2(p.ws_m[base + k] - M) : 0.f;
    den = fmaf(w, lk, den);
    num = fmaf(w, p.ws_acc[(base + k) * D + threadIdx.x], num);
  }
  QS* o = reinterpret_cast<QS*>(ptr.out) + (size_t(s) * p.H + h) * D;
  o[threadIdx.x] = from_f32<QDT>(den > 0.f ? num * (p.v_scale / den) : 0.f);
}

template <DT Q, DT C, int D>
hipError_t run_valu(const DecodePtrs& ptr, const DecodeParams& p, hipStream_t stream) {
  const long long units = 1LL * p.np * p.S * p.H;
  hipLaunchKernelGGL((decode_valu_kernel<Q, C, D>), dim3(unsigned(units)), dim3(64), 0, stream,
                     ptr, p);
  return hipGetLastError();
}

template <DT Q, int D>
hipError_t run_merge(const DecodePtrs& ptr, const DecodeParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((merge_kernel<Q, D>), dim3(unsigned(p.S * p.H)), dim3(D), 0, stream, ptr, p);
  return hipGetLastError();
}

template <DT Q, DT C>
hipError_t by_d(int D, const DecodePtrs& ptr, const DecodeParams& p, hipStream_t st) {
  return D == 64 ? run_valu<Q, C, 64>(ptr, p, st) : run_valu<Q, C, 128>(ptr, p, st);
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
  if (q == DT::F32) return D == 64 ? run_merge<DT::F32, 64>(ptr, p, stream)
                                   : run_merge<DT::F32, 128>(ptr, p, stream);
  if (q == DT::F16) return D == 64 ? run_merge<DT::F16, 64>(ptr, p, stream)
                                   : run_merge<DT::F16, 128>(ptr, p, stream);
  return D == 64 ? run_merge<DT::BF16, 64>(ptr, p, stream)
                 : run_merge<DT::BF16, 128>(ptr, p, stream);
}

}  // namespace pkv
