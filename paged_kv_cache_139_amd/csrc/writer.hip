// Slot-mapped KV writer and the block-table gather.
//
// reshape_and_cache: each new token's key/value row [Hk, D] (token t's row
// at element t * key_stride / t * value_stride of the source) is stored into
// the paged caches at slot = block * BLOCK_SIZE + offset ([TGI] §4.1, the KV
// write side, bit copy or FP8 quantised write).  One thread moves 8
// consecutive head_size elements of one (token, head): a 16- or 32-byte
// contiguous read of the source and 8 writes strided by the block's row of
// BLOCK_SIZE tokens (BLOCK_SIZE = 1 << lbs).
//
// paged_kv_gather: the logical KV of one sequence through its block table
// ([L3] "SVG框架图"), bits unchanged.
#include <type_traits>

#include "device_common.h"

namespace pkv {
namespace {

template <DT SRC, DT CACHE>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const uint8_t* __restrict__ key, const uint8_t* __restrict__ value, uint8_t* __restrict__ kc,
    uint8_t* __restrict__ vc, const int64_t* __restrict__ slots, int T, int Hk, int D, int NB,
    int lbs, long long key_stride, long long value_stride, float k_scale, float v_scale) {
  using SS = typename Elem<SRC>::storage;
  using CS = typename Elem<CACHE>::storage;
  const int chunks = D / 8;
  const long long item = 1LL * blockIdx.x * blockDim.x + threadIdx.x;
  if (item >= 1LL * T * Hk * chunks) return;
  const int c = int(item % chunks);
  const int h = int((item / chunks) % Hk);
  const int t = int(item / (1LL * chunks * Hk));
  const long long slot = slots[t];
  const int bs = 1 << lbs;
  if (slot < 0 || slot >= (1LL * NB) << lbs) return;
  const long long b = slot >> lbs;
  const int o = int(slot & (bs - 1));

  const size_t in_row = size_t(h) * D + size_t(c) * 8;                  // elements
  const size_t dst = (((size_t(b) * Hk + h) * D + size_t(c) * 8) << lbs) + o;
  const SS* ks = reinterpret_cast<const SS*>(key) + size_t(t) * key_stride + in_row;
  const SS* vs = reinterpret_cast<const SS*>(value) + size_t(t) * value_stride + in_row;
  CS* kd = reinterpret_cast<CS*>(kc) + dst;
  CS* vd = reinterpret_cast<CS*>(vc) + dst;

  if constexpr (SRC == CACHE) {
    // integer words: a pure bit copy, NaN payloads included
    using W = typename std::conditional<sizeof(SS) == 4, uint32_t, uint16_t>::type;
    const W* kw = reinterpret_cast<const W*>(ks);
    const W* vw = reinterpret_cast<const W*>(vs);
    W kv[8], vv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kv[e] = kw[e];
      vv[e] = vw[e];
    }
    W* kdw = reinterpret_cast<W*>(kd);
    W* vdw = reinterpret_cast<W*>(vd);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kdw[e * bs] = kv[e];
      vdw[e * bs] = vv[e];
    }
  } else {
    static_assert(CACHE == DT::FP8);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // one correctly rounded float32 division, then E4M3 rounding
      kd[e * bs] = uint8_t(f32_to_e4m3(__fdiv_rn(load_f32<SRC>(ks + e), k_scale)));
      vd[e * bs] = uint8_t(f32_to_e4m3(__fdiv_rn(load_f32<SRC>(vs + e), v_scale)));
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

template <DT S, DT C>
hipError_t run_writer(const void* key, const void* value, void* kc, void* vc, const int64_t* slots,
                      int T, int Hk, int D, int NB, int lbs, long long kst, long long vst,
                      float ks, float vs, hipStream_t stream) {
  const long long items = 1LL * T * Hk * (D / 8);
  const unsigned grid = unsigned((items + 255) / 256);
  hipLaunchKernelGGL((reshape_and_cache_kernel<S, C>), dim3(grid), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(key), static_cast<const uint8_t*>(value),
                     static_cast<uint8_t*>(kc), static_cast<uint8_t*>(vc), slots, T, Hk, D, NB,
                     lbs, kst, vst, ks, vs);
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
