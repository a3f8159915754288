// a4 - gather attention over the position buffer.
//
// The arex-research.com article (section on the four optimisations, item 3)
// describes a sparse attention kernel for normal decode and MTP verify with
// BF16 queries and BF16 or FP8 E4M3 KV.  This is a gfx950 design for the same
// contract.
//
// Work unit: (query, split of the position buffer, KV head) = grid (x, y, z).  A wave takes
// 32 gathered positions per step and serves the whole GQA group of that KV
// head (up to 16 query heads) at once on bf16 MFMA 16x16x32:
//   S^T[pos][head] = K[pos][:] . Q[head][:]      (2 tiles x 4 MFMAs)
//   O^T[dim][head] += V^T[dim][pos] P^T[pos][head]  (8 MFMAs each for the BF16
//                                                    high and low parts of P)
// The GQA group is the 16-column side of the tile; the gathered positions
// are the dense side.  The position order inside the k dimension of the PV
// product is chosen so that each lane's P values come straight out of the
// S^T accumulator registers, and each lane gathers exactly the V rows its own
// P values need (16 contiguous bytes per row), repacked with byte permutes -
// no LDS round trip.  FP8 E4M3FN rows are widened exactly to BF16 with the
// hardware converter; the per-head K scale folds into the softmax scale and
// the V scale into the final normalisation.
//
// Softmax is online per wave (running max and sum in the log2 domain), the 4
// waves of a workgroup merge in LDS, and when a unit is split over several
// workgroups the last one to finish merges the partials (an arrival counter
// in the workspace, one 128-byte line per unit, reset to zero by that last
// workgroup).  Partials travel through device-coherent stores and loads, so
// the hand-off needs no cache flush or invalidation.
#include "qsa_common.hpp"
#include "qsa_launch.hpp"

namespace qsa {

constexpr int kOStride = QSA_HEAD_DIM + 4;   // padded LDS row of one head's output

struct AttnParams {
  const uint16_t* q;
  const uint8_t* kc;
  const uint8_t* vc;
  const float* k_scale;
  const float* v_scale;
  const int32_t* pos;
  const int32_t* n_pos;
  void* out;
  float* part;
  uint32_t* counters;
  int width, num_q_heads, num_kv_heads, group;
  float sm_scale_log2;
  int splits, cps;
};

__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// 4 FP8 E4M3FN bytes -> 4 BF16 (exact), as 2 packed dwords (low bytes first).
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t w) {
  return u32x2{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true))};
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <bool kFp8, bool kOutBf16>
__global__ __launch_bounds__(256) void attn_kernel(AttnParams p) {
  constexpr int D = QSA_HEAD_DIM;
  constexpr int EB = kFp8 ? 1 : 2;            // bytes per KV element
  __shared__ float o_s[kAttnWaves][16][kOStride];
  __shared__ float m_s[kAttnWaves][16], l_s[kAttnWaves][16];
  __shared__ float w_s[16];
  __shared__ float ml_s[kMaxSplits][32];
  __shared__ int s_last;

  const int q = blockIdx.x, s = blockIdx.y, g = blockIdx.z;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int j = lane & 15, kg = lane >> 4;
  const int G = p.group;
  const bool hvalid = j < G;
  const int Hq = p.num_q_heads, Hkv = p.num_kv_heads;

  const int npos = p.n_pos[q];
  const int nchunks = (npos + kChunk - 1) / kChunk;
  const int c_begin = s * p.cps;
  const int c_end = min(c_begin + p.cps, nchunks);
  const int32_t* prow = p.pos + (int64_t)q * p.width;
  const int slot0 = prow[0];

  // Q^T as the B operand: lane (kg, j) holds head j, dims kg*32 + kk*8 + e.
  bf16x8 qb[4];
  {
    const uint16_t* qrow = p.q + ((int64_t)q * Hq + g * G + j) * D + kg * 32;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u32x4 v = hvalid ? *reinterpret_cast<const u32x4*>(qrow + kk * 8) : u32x4{0u, 0u, 0u, 0u};
      qb[kk] = __builtin_bit_cast(bf16x8, v);
    }
  }
  const float kscale = kFp8 ? p.k_scale[g] : 1.f;
  const float vscale = kFp8 ? p.v_scale[g] : 1.f;
  const float sl2 = p.sm_scale_log2 * kscale;
  const int64_t row_stride = (int64_t)Hkv * D * EB;   // bytes between consecutive slots
  const uint8_t* kbase = p.kc + (int64_t)g * D * EB;
  const uint8_t* vbase = p.vc + (int64_t)g * D * EB;

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) o[u] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int c = c_begin + wave; c < c_end; c += kAttnWaves) {
    const int base = c * kChunk;
    // K rows: position 16t + j of the chunk; V rows: positions 16t + 4kg + rr.
    int ks[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int idx = base + 16 * t + j;
      const int sl = idx < npos ? prow[idx] : -1;
      ks[t] = sl >= 0 ? sl : slot0;
    }
    int vs[8];
    bool valid[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int idx = base + 16 * (e >> 2) + 4 * kg + (e & 3);
      const int sl = idx < npos ? prow[idx] : -1;
      valid[e] = sl >= 0;
      vs[e] = sl >= 0 ? sl : slot0;
    }

    // K operand (A): lane holds dims kg*32 .. kg*32+31 of its row, as 4 x 8 bf16.
    bf16x8 ka[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint8_t* kr = kbase + (int64_t)ks[t] * row_stride + kg * 32 * EB;
      if (kFp8) {
        const u32x4 w0 = *reinterpret_cast<const u32x4*>(kr);
        const u32x4 w1 = *reinterpret_cast<const u32x4*>(kr + 16);
        const uint32_t ws[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const u32x2 lo = fp8x4_to_bf16x4(ws[2 * kk]), hi = fp8x4_to_bf16x4(ws[2 * kk + 1]);
          ka[t][kk] = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
        }
      } else {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          ka[t][kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kr + kk * 16));
      }
    }
    // V rows: dims 8j .. 8j+7 of each of the lane's 8 positions, as 8 bf16.
    u32x4 vr[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint8_t* vp = vbase + (int64_t)vs[e] * row_stride + j * 8 * EB;
      if (kFp8) {
        const u32x2 w = *reinterpret_cast<const u32x2*>(vp);
        const u32x2 lo = fp8x4_to_bf16x4(w.x), hi = fp8x4_to_bf16x4(w.y);
        vr[e] = u32x4{lo.x, lo.y, hi.x, hi.y};
      } else {
        vr[e] = *reinterpret_cast<const u32x4*>(vp);
      }
    }

    // S^T = K Q^T: accumulator row kg*4 + rr = position 16t + 4kg + rr, column j = head.
    f32x4 sacc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[t][kk], qb[kk], sacc[t], 0, 0, 0);
    }
    float sv[8];
    float mloc = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sv[e] = valid[e] ? sacc[e >> 2][e & 3] * sl2 : -INFINITY;
      mloc = fmaxf(mloc, sv[e]);
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16, kWave));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, kWave));
    const float m_new = fmaxf(m_run, mloc);
    const float alpha = exp2f(m_run - m_new);
    // P = P_hi + P_lo, both BF16: the PV product then carries ~16 bits of P.
    uint32_t ph[4], plo[4];
    float psum = 0.f;
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      const float p0 = exp2f(sv[2 * e2] - m_new), p1 = exp2f(sv[2 * e2 + 1] - m_new);
      ph[e2] = pack_bf16x2(p0, p1);
      plo[e2] = pack_bf16x2(p0 - bf16lo_to_f32(ph[e2]), p1 - bf16hi_to_f32(ph[e2]));
      psum += p0 + p1;
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    const bf16x8 pb_hi = __builtin_bit_cast(bf16x8, u32x4{ph[0], ph[1], ph[2], ph[3]});
    const bf16x8 pb_lo = __builtin_bit_cast(bf16x8, u32x4{plo[0], plo[1], plo[2], plo[3]});

    // O^T += V^T P^T; tile u covers dims 8i + u for accumulator row i.
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t selb = (u & 1) ? 0x07060302u : 0x05040100u;
      u32x4 a;
      a.x = perm_b32(vr[1][u >> 1], vr[0][u >> 1], selb);
      a.y = perm_b32(vr[3][u >> 1], vr[2][u >> 1], selb);
      a.z = perm_b32(vr[5][u >> 1], vr[4][u >> 1], selb);
      a.w = perm_b32(vr[7][u >> 1], vr[6][u >> 1], selb);
      const bf16x8 va = __builtin_bit_cast(bf16x8, a);
      o[u] = o[u] * alpha;
      o[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb_hi, o[u], 0, 0, 0);
      o[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb_lo, o[u], 0, 0, 0);
    }
  }

  // Row sums over the 4 lane groups of a head.
  l_run += __shfl_xor(l_run, 16, kWave);
  l_run += __shfl_xor(l_run, 32, kWave);

  // Lane (kg, j) holds O[head j][32kg + 8rr + u] = o[u][rr].
  if (hvalid) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      float* dst = &o_s[wave][j][32 * kg + 8 * rr];
      *reinterpret_cast<f32x4*>(dst) = f32x4{o[0][rr], o[1][rr], o[2][rr], o[3][rr]};
      *reinterpret_cast<f32x4*>(dst + 4) = f32x4{o[4][rr], o[5][rr], o[6][rr], o[7][rr]};
    }
    if (kg == 0) {
      m_s[wave][j] = m_run;
      l_s[wave][j] = l_run;
    }
  }
  __syncthreads();

  const int nout = G * D;
  if (p.splits == 1) {
    for (int idx = tid; idx < nout; idx += blockDim.x) {
      const int hh = idx / D, d = idx % D;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, m_s[w][hh]);
      float num = 0.f, den = 0.f;
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) {
        const float sc = m_s[w][hh] == -INFINITY ? 0.f : exp2f(m_s[w][hh] - M);
        num += sc * o_s[w][hh][d];
        den += sc * l_s[w][hh];
      }
      const float val = num / den * vscale;
      const int64_t oi = ((int64_t)q * Hq + g * G + hh) * D + d;
      if (kOutBf16) static_cast<__bf16*>(p.out)[oi] = (__bf16)val;
      else static_cast<float*>(p.out)[oi] = val;
    }
    return;
  }

  // Split partial: [G*128 unnormalised O][16 m][16 l] per (q, g, s), published
  // with device-coherent (write-through) stores: no cache flush is needed
  // before the arrival is counted, only the stores' completion.
  const int pstride = G * D + 32;
  float* unit = p.part + ((int64_t)q * Hkv + g) * p.splits * pstride;
  float* mine = unit + (int64_t)s * pstride;
  for (int idx = tid; idx < nout + 2 * G; idx += blockDim.x) {
    float val;
    int dst;
    if (idx < nout) {
      const int hh = idx / D, d = idx % D;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, m_s[w][hh]);
      float num = 0.f;
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w)
        num += (m_s[w][hh] == -INFINITY ? 0.f : exp2f(m_s[w][hh] - M)) * o_s[w][hh][d];
      val = num;
      dst = idx;
    } else {
      const int hh = (idx - nout) % G;
      const bool is_l = (idx - nout) >= G;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, m_s[w][hh]);
      if (!is_l) {
        val = M;
        dst = nout + hh;
      } else {
        float den = 0.f;
#pragma unroll
        for (int w = 0; w < kAttnWaves; ++w)
          den += (m_s[w][hh] == -INFINITY ? 0.f : exp2f(m_s[w][hh] - M)) * l_s[w][hh];
        val = den;
        dst = nout + 16 + hh;
      }
    }
    __hip_atomic_store(mine + dst, val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0);     // this thread's stores have reached the coherence point
  __syncthreads();
  if (tid == 0) {
    const uint32_t ticket = atomicAdd(&p.counters[(q * Hkv + g) * kCounterStride], 1u);
    s_last = ticket == (uint32_t)(p.splits - 1);
  }
  __syncthreads();
  if (!s_last) return;

  // Last workgroup of the unit: merge all splits with device-coherent loads.
  const int S = p.splits;
  for (int i = tid; i < S * 2 * G; i += blockDim.x) {
    const int t = i / (2 * G), r = i % (2 * G);
    const int off = r < G ? nout + r : nout + 16 + (r - G);
    ml_s[t][r] = __hip_atomic_load(unit + (int64_t)t * pstride + off, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (tid < G) {
    float M = -INFINITY;
    for (int t = 0; t < S; ++t) M = fmaxf(M, ml_s[t][tid]);
    float den = 0.f;
    for (int t = 0; t < S; ++t) {
      const float mt = ml_s[t][tid];
      const float wgt = mt == -INFINITY ? 0.f : exp2f(mt - M);
      ml_s[t][tid] = wgt;                       // weight of split t for head tid
      den += wgt * ml_s[t][G + tid];
    }
    w_s[tid] = vscale / den;
  }
  __syncthreads();
  for (int idx = tid; idx < nout; idx += blockDim.x) {
    const int hh = idx / D;
    float vals[kMaxSplits];
#pragma unroll
    for (int t = 0; t < kMaxSplits; ++t)
      vals[t] = t < S ? __hip_atomic_load(unit + (int64_t)t * pstride + idx, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT)
                      : 0.f;
    float num = 0.f;
#pragma unroll
    for (int t = 0; t < kMaxSplits; ++t)
      if (t < S) num += ml_s[t][hh] * vals[t];
    const float val = num * w_s[hh];
    const int64_t oi = ((int64_t)q * Hq + g * G) * D + idx;
    if (kOutBf16) static_cast<__bf16*>(p.out)[oi] = (__bf16)val;
    else static_cast<float*>(p.out)[oi] = val;
  }
  if (tid == 0) p.counters[(q * Hkv + g) * kCounterStride] = 0u;
}

size_t attn_partial_bytes(int num_q, int num_kv_heads, int group, int width) {
  const AttnSplit sp = attn_split(num_q, num_kv_heads, width);
  if (sp.splits <= 1) return 0;
  return (size_t)num_q * num_kv_heads * sp.splits * (group * QSA_HEAD_DIM + 32) * sizeof(float);
}

hipError_t launch_attn(const Meta& m, const AttnArgs& a, hipStream_t stream) {
  const AttnSplit sp = attn_split(m.num_q, a.num_kv_heads, a.width);
  AttnParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.kc = static_cast<const uint8_t*>(a.k_cache);
  p.vc = static_cast<const uint8_t*>(a.v_cache);
  p.k_scale = a.k_scale;
  p.v_scale = a.v_scale;
  p.pos = a.pos;
  p.n_pos = a.n_pos;
  p.out = a.out;
  p.part = a.partials;
  p.counters = a.counters;
  p.width = a.width;
  p.num_q_heads = a.num_q_heads;
  p.num_kv_heads = a.num_kv_heads;
  p.group = a.num_q_heads / a.num_kv_heads;
  p.sm_scale_log2 = a.sm_scale * 1.4426950408889634f;
  p.splits = sp.splits;
  p.cps = sp.chunks_per_split;
  dim3 grid((unsigned)m.num_q, (unsigned)sp.splits, (unsigned)a.num_kv_heads);
  if (a.kv_fp8) {
    if (a.out_bf16) attn_kernel<true, true><<<grid, 256, 0, stream>>>(p);
    else attn_kernel<true, false><<<grid, 256, 0, stream>>>(p);
  } else {
    if (a.out_bf16) attn_kernel<false, true><<<grid, 256, 0, stream>>>(p);
    else attn_kernel<false, false><<<grid, 256, 0, stream>>>(p);
  }
  return hipGetLastError();
}

}  // namespace qsa
