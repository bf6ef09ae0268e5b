// Core multi-query attention over compressed entries plus the sliding window, with a per-head sink
// (page 1, "hybrid attention": CSA step 3, the HCA paragraph, Q/KV normalization, partial RoPE with
// the output rotated by -i, the sliding-window branch, the attention sink; page 4 section 3.1).
//
// For a query at token t and head h:  qhat = RoPE_t(RMSNorm(q_h)),  l_j = scale * qhat . k_j,
// o_h = sum_j e^{l_j} k_j / (e^{z_h} + sum_j e^{l_j})  (K = V),  then o_h[448:] rotated by -t.
// Keys: the selected entries (CSA) or every visible entry (HCA), followed by tokens [t-W+1, t].
//
// All query heads share each 1 KiB K=V row, so per key the work is 64 heads x 512 dims twice
// (QK^T and PV): ~128 flop per byte, above the fp32-vector ridge, hence bf16 MFMA for both.
// Workgroup = 4 waves; wave w owns dims [128w, 128w+128) of every key, for all heads:
//   - its K slice comes straight from HBM into MFMA A-fragments (16 B loads, 256 B per key),
//   - partial logits over its 128 dims are summed across the 4 waves through LDS,
//   - wave w' < HB runs the online softmax of head block w' and publishes P (bf16) and the
//     rescale factors,
//   - every wave then accumulates O[:, its 128 dims] += P V with V read back from its own LDS copy
//     of the slice, laid out so the k-major V fragment reads hit 32 distinct banks.
// Keys are split across workgroups (split-K); partial (max, sum, O) are merged by merge_kernel,
// which adds the sink once.  With one split the workgroup finishes the output itself.
#include "common.h"
#include "kernels.h"

namespace lcs {

namespace {

constexpr int kTile = 32;                 // keys per tile
constexpr int kMaxSplitKeys = 2048;       // keys of one split, staged as row indices in LDS
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4 GU32x4;   // global address space: global_load, not flat
constexpr int kVtStride = 136;            // bf16 per LDS row of the V slice (128 + 8 pad)
constexpr float kLog2e = 1.4426950408889634f;

struct AttnK {
  const uint16_t* q; const uint16_t* gamma_q;
  const uint16_t* kv; int64_t kv_ld;
  const int32_t* topk; int k;
  int64_t n_cap; int m;
  const uint16_t* win; int64_t win_ld, ring_cap; int window;
  const float* sink; const int64_t* q_pos; int64_t rope_offset;
  int Tq, H; float scale_log2, eps;
  RopeFreq rf;
  uint16_t* out; uint16_t* part_o; float* part_ml;
  int nsplit, keys_per_split, hgroups;
};

struct RowKeys {
  int64_t t, nc, nk;                      // query token, compressed keys in the list, total keys
};

// LDS row of the V-slice copy for tile key (block kb, row r16 of the 16x16 MFMA block).
__device__ __forceinline__ int vt_row(int kb, int r16) { return 2 * (r16 >> 2) + 8 * (r16 & 3) + kb; }

template <int HB>
__global__ void __launch_bounds__(256, 1)
attend_kernel(AttnK a) {
  __shared__ float4 s_part[4 * 2 * HB * kWave];            // partial logits [wave][kb][hb][lane]
  __shared__ uint4 s_q[4][HB][4][kWave];                    // qhat fragments [wave][hb][ks][lane]
  __shared__ uint16_t s_vt[4][kTile * kVtStride];         // per-wave V slice
  __shared__ uint4 s_p[HB * kWave];                        // P fragments [hb][lane]
  __shared__ float s_alpha[HB * 16];
  __shared__ float s_fac[HB * 16];
  __shared__ float s_ssq[4][HB * 16];
  __shared__ float s_cos[32], s_sin[32];
  __shared__ int s_nsel;
  __shared__ int32_t s_rows[kMaxSplitKeys];                 // per key of this split: cache/ring row, -1 = none
  __shared__ int s_rescale[2];            // per tile parity: some head's reference max moved

  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  const int g = lane >> 4, c16 = lane & 15;
  const int64_t r = blockIdx.y;
  const int64_t b = r / a.Tq;
  // Block ids are grouped 8 at a time so that the head-group workgroups of one split have ids 8 apart
  // and therefore run on the same XCD (workgroups are dealt to the 8 XCDs round-robin): the second
  // one finds the key tiles in that XCD's L2.
  const int bid = blockIdx.x;
  const int grp = bid / (8 * a.hgroups), rem = bid % (8 * a.hgroups);
  const int split = grp * 8 + rem % 8;
  if (split >= a.nsplit) return;                           // padding workgroup (uniform)
  const int head0 = (rem / 8) * 16 * HB;

  if (threadIdx.x == 0) { s_rescale[0] = 0; s_rescale[1] = 0; }
  RowKeys rk;
  rk.t = a.q_pos[r];
  if (a.topk) {
    // compressed keys in the list: up to the last non-negative index
    if (threadIdx.x == 0) s_nsel = 0;
    __syncthreads();
    int last = 0;
    constexpr int kPer = 2048 / 256;     // k <= 2048: all loads in flight together
    int32_t v[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = threadIdx.x + 256 * u;
      v[u] = a.topk[r * a.k + (i < a.k ? i : 0)];
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = threadIdx.x + 256 * u;
      if (i < a.k && v[u] >= 0) last = i + 1;
    }
    atomicMax(&s_nsel, last);
    __syncthreads();
    rk.nc = s_nsel;
  } else {
    int64_t nv = rk.t >= 0 ? rk.t / a.m : 0;
    rk.nc = nv < a.n_cap ? nv : a.n_cap;
  }
  rk.nk = rk.nc + a.window;
  const int64_t e_begin = (int64_t)split * a.keys_per_split;
  int64_t e_end = e_begin + a.keys_per_split;
  if (e_end > rk.nk) e_end = rk.nk;

  // rope table for this query position (same angles for every head)
  const double pos = (double)(rk.t + a.rope_offset);
  if (threadIdx.x < 32) {
    float cs, sn;
    rope_cs(pos, a.rf.inv[threadIdx.x], &cs, &sn);
    s_cos[threadIdx.x] = cs;
    s_sin[threadIdx.x] = sn;
  }

  const int ntiles = e_end > e_begin ? (int)((e_end - e_begin + kTile - 1) / kTile) : 0;

  // ---- the split's key rows, staged once: compressed keys (selected index or entry number), then
  //      window tokens (ring row), -1 where a key does not exist ----
  const int nkeys = e_end > e_begin ? (int)(e_end - e_begin) : 0;
  {
    const int64_t j0 = rk.t - a.window + 1;               // first window token
    constexpr int kPer = kMaxSplitKeys / 256;
    int32_t sel[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {                     // the selected indices: one round trip
      const int64_t e = e_begin + threadIdx.x + 256 * u;
      sel[u] = a.topk ? a.topk[r * a.k + (e < rk.nc ? e : 0)] : 0;   // unconditional (clamped) load
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = threadIdx.x + 256 * u;
      if (i < nkeys) {
        const int64_t e = e_begin + i;
        int32_t row;
        if (e < rk.nc) {
          row = a.topk ? sel[u] : (int32_t)e;
        } else {
          const int64_t j = j0 + (e - rk.nc);
          row = j < 0 ? -1 : (int32_t)(a.ring_cap > 0 ? j % a.ring_cap : j);
        }
        s_rows[i] = row;
      }
    }
  }
  __syncthreads();
  const uint16_t* kv_b = a.kv + b * a.kv_ld * kHeadDim;
  const uint16_t* win_b = a.win ? a.win + b * a.win_ld * kHeadDim : a.kv;
  const int nc_local = rk.nc > e_begin ? (int)(rk.nc - e_begin) : 0;   // split keys that are compressed

  // ---- tile loads: this lane feeds MFMA rows kb*16 + c16 ----
  uint4 kcur[2][4];
  uint32_t vcur = 0;
  auto load_tile = [&](int i0, uint4 (&kf)[2][4], uint32_t& vmask) {
    const int i = i0 + (lane & 31);
    const int32_t row = i < nkeys ? s_rows[i] : -1;
    vmask = (uint32_t)__ballot(row >= 0 && lane < 32);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int src = kb * 16 + c16;
      const int32_t rr = __shfl(row, src, kWave);
      const uint16_t* base = (i0 + src) < nc_local ? kv_b : win_b;
      // always a readable row (row 0 when the key does not exist): no predicated loads
      GU32x4* p = reinterpret_cast<GU32x4*>(reinterpret_cast<uintptr_t>(base + (int64_t)(rr > 0 ? rr : 0) * kHeadDim +
                                                                          128 * w + 8 * g));
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {                         // invalid keys are zeroed where consumed
        const u32x4 x = p[4 * ks];
        kf[kb][ks] = make_uint4(x.x, x.y, x.z, x.w);
      }
    }
  };
  if (ntiles > 0) load_tile(0, kcur, vcur);                // first tile in flight during the q prologue

  // ---- qhat fragments: B operand of S^T = K qhat^T, lane holds head c16 of block hb,
  //      dims 128w + 32ks + 8g .. +8 ----
  uint4 qf[HB][4];
  {
    float ss[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const int head = head0 + hb * 16 + c16;
      const bool hv = head < a.H;
      const int hl = hv ? head : a.H - 1;
      float acc = 0.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int d = 128 * w + 32 * ks + 8 * g;
        uint4 x = *reinterpret_cast<const uint4*>(a.q + (r * a.H + hl) * kHeadDim + d);
        if (!hv) x = make_uint4(0, 0, 0, 0);
        qf[hb][ks] = x;
        const float v[8] = {bf2f_lo(x.x), bf2f_hi(x.x), bf2f_lo(x.y), bf2f_hi(x.y),
                            bf2f_lo(x.z), bf2f_hi(x.z), bf2f_lo(x.w), bf2f_hi(x.w)};
#pragma unroll
        for (int j = 0; j < 8; ++j) acc += v[j] * v[j];
      }
      acc += __shfl_xor(acc, 16, kWave);
      acc += __shfl_xor(acc, 32, kWave);
      ss[hb] = acc;
      if (g == 0) s_ssq[w][hb * 16 + c16] = acc;
    }
    uint4 gmv[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) gmv[ks] = *reinterpret_cast<const uint4*>(a.gamma_q + 128 * w + 32 * ks + 8 * g);
    __syncthreads();
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const float tot = s_ssq[0][hb * 16 + c16] + s_ssq[1][hb * 16 + c16] + s_ssq[2][hb * 16 + c16] +
                        s_ssq[3][hb * 16 + c16];
      const float rstd = 1.0f / sqrtf(tot * (1.0f / kHeadDim) + a.eps);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int d = 128 * w + 32 * ks + 8 * g;
        const uint4 x = qf[hb][ks];
        const uint4 gm = gmv[ks];
        float v[8] = {bf2f_lo(x.x), bf2f_hi(x.x), bf2f_lo(x.y), bf2f_hi(x.y),
                      bf2f_lo(x.z), bf2f_hi(x.z), bf2f_lo(x.w), bf2f_hi(x.w)};
        const float gv[8] = {bf2f_lo(gm.x), bf2f_hi(gm.x), bf2f_lo(gm.y), bf2f_hi(gm.y),
                             bf2f_lo(gm.z), bf2f_hi(gm.z), bf2f_lo(gm.w), bf2f_hi(gm.w)};
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = v[j] * rstd * gv[j];
        if (d >= kRopeStart) {
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const int jr = (d + 2 * p - kRopeStart) >> 1;
            const float cs = s_cos[jr], sn = s_sin[jr];
            const float a0 = v[2 * p], a1 = v[2 * p + 1];
            v[2 * p] = a0 * cs - a1 * sn;
            v[2 * p + 1] = a0 * sn + a1 * cs;
          }
        }
        s_q[w][hb][ks][lane] = make_uint4(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]), pack_bf2(v[4], v[5]),
                                pack_bf2(v[6], v[7]));
      }
    }
    (void)ss;
  }

  floatx4 o[HB][8];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb)
#pragma unroll
    for (int db = 0; db < 8; ++db) o[hb][db] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;      // softmax state of head (16w + c16), waves w < HB

  // One 32-key tile: QK^T partials, softmax, PV.  kf holds the tile's fragments, vm its key mask.
  auto process = [&](uint4 (&kf)[2][4], uint32_t vm, int it) {
    // opaque zero: keeps the qhat fragment reads inside the tile (hoisting them would pin 16*HB
    // registers for the whole loop)
    int qz;
    asm volatile("v_mov_b32 %0, 0" : "=v"(qz));

    // zero the rows of invalid keys (their loads read a real row so that no load is predicated)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bool v = (vm >> (kb * 16 + c16)) & 1u;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kf[kb][ks] = v ? kf[kb][ks] : make_uint4(0, 0, 0, 0);
    }
    // partial S^T over this wave's 128 dims
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc = mfma_bf16(kf[kb][ks], s_q[w][hb][ks][lane + qz], acc);
        s_part[((w * 2 + kb) * HB + hb) * kWave + lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      }
      const int vr = vt_row(kb, c16);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        *reinterpret_cast<uint4*>(&s_vt[w][vr * kVtStride + 32 * ks + 8 * g]) = kf[kb][ks];
    }
    __syncthreads();

    if (w < HB) {
      float s[2][4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float4 t0 = s_part[((0 * 2 + kb) * HB + w) * kWave + lane];
        float4 t1 = s_part[((1 * 2 + kb) * HB + w) * kWave + lane];
        float4 t2 = s_part[((2 * 2 + kb) * HB + w) * kWave + lane];
        float4 t3 = s_part[((3 * 2 + kb) * HB + w) * kWave + lane];
        s[kb][0] = (t0.x + t1.x) + (t2.x + t3.x);
        s[kb][1] = (t0.y + t1.y) + (t2.y + t3.y);
        s[kb][2] = (t0.z + t1.z) + (t2.z + t3.z);
        s[kb][3] = (t0.w + t1.w) + (t2.w + t3.w);
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool v = (vm >> (kb * 16 + 4 * g + i)) & 1u;
          s[kb][i] = v ? s[kb][i] * a.scale_log2 : -INFINITY;
          tmax = fmaxf(tmax, s[kb][i]);
        }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
      // Lazy rescaling: the reference max only moves when the tile max exceeds it by more than
      // 2^8 (p then stays <= 256, exact in the fp32 sums and in bf16's exponent range); the
      // final normalisation uses the same reference, so the result is unchanged.
      float m_new = m_run;
      float alpha = 1.f;
      if (m_run == -INFINITY) {
        m_new = tmax;                      // nothing accumulated yet: O and l are zero
      } else if (tmax > m_run + 8.f) {
        m_new = tmax;
        alpha = exp2f(m_run - m_new);
        s_rescale[it & 1] = 1;
      }
      if (w == 0 && lane == 0) s_rescale[(it + 1) & 1] = 0;   // read last by the previous tile's PV
      uint32_t pk[4] = {0u, 0u, 0u, 0u};
      float psum = 0.f;
      if (m_new != -INFINITY) {
        float p[8];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) p[kb * 4 + i] = exp2f(s[kb][i] - m_new);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pk[j] = pack_bf2(p[2 * j], p[2 * j + 1]);
          psum += bf2f_lo(pk[j]) + bf2f_hi(pk[j]);
        }
      }
      psum += __shfl_xor(psum, 16, kWave);
      psum += __shfl_xor(psum, 32, kWave);
      l_run = l_run * alpha + psum;
      m_run = m_new;
      s_p[w * kWave + lane] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
      if (g == 0) s_alpha[w * 16 + c16] = alpha;
    }
    __syncthreads();

    if (s_rescale[it & 1]) {               // rare: some head's reference max moved this tile
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        const float4 al = *reinterpret_cast<const float4*>(&s_alpha[hb * 16 + 4 * g]);
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          o[hb][db][0] *= al.x;
          o[hb][db][1] *= al.y;
          o[hb][db][2] *= al.z;
          o[hb][db][3] *= al.w;
        }
      }
    }
    uint4 pf[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) pf[hb] = s_p[hb * kWave + lane];
    const uint16_t* vt = s_vt[w];
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int col = 16 * db + c16;
      uint32_t vv[4];
#pragma unroll
      for (int j2 = 0; j2 < 4; ++j2) {
        const int j0 = 2 * j2, j1 = 2 * j2 + 1;
        const uint32_t lo = vt[(2 * g + 8 * (j0 & 3) + (j0 >> 2)) * kVtStride + col];
        const uint32_t hi = vt[(2 * g + 8 * (j1 & 3) + (j1 >> 2)) * kVtStride + col];
        vv[j2] = lo | (hi << 16);
      }
      const uint4 vf = make_uint4(vv[0], vv[1], vv[2], vv[3]);
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) o[hb][db] = mfma_bf16(pf[hb], vf, o[hb][db]);
    }

  };

  // Two register buffers rotate by unrolling (a copy between buffers would wait for the loads in
  // flight): the next tile's loads are in flight while the current one is processed.  A load past
  // the end re-reads the last tile (never processed).
  uint4 k1[2][4];
  uint32_t v1 = 0;
  auto tile0 = [&](int t) { return (t < ntiles ? t : ntiles - 1) * kTile; };
  if (ntiles > 0) {
    for (int t = 0; t < ntiles; t += 2) {
      load_tile(tile0(t + 1), k1, v1);
      __builtin_amdgcn_sched_barrier(0);
      process(kcur, vcur, t);
      __builtin_amdgcn_sched_barrier(0);
      if (t + 1 >= ntiles) break;
      load_tile(tile0(t + 2), kcur, vcur);
      __builtin_amdgcn_sched_barrier(0);
      process(k1, v1, t + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  if (a.nsplit == 1) {
    // finish here: add the sink, normalise, rotate the last 64 dims by -(t + offset), store bf16
    if (w < HB) {
      const int head = head0 + w * 16 + c16;
      const float z = head < a.H ? a.sink[head] * kLog2e : -INFINITY;
      const float M = fmaxf(m_run, z);
      float f = 0.f;
      if (M != -INFINITY) {
        const float L = l_run * exp2f(m_run - M) + exp2f(z - M);
        f = exp2f(m_run - M) / L;
      }
      if (g == 0) s_fac[w * 16 + c16] = f;
    }
    __syncthreads();
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const int d = 128 * w + 16 * db + c16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int hl = hb * 16 + 4 * g + i;
          float v = o[hb][db][i] * s_fac[hl];
          const float pv = __shfl_xor(v, 1, kWave);
          if (d >= kRopeStart) {
            const int jr = (d - kRopeStart) >> 1;
            const float cs = s_cos[jr], sn = s_sin[jr];
            v = (c16 & 1) ? (-pv * sn + v * cs) : (v * cs + pv * sn);
          }
          const int head = head0 + hl;
          if (head < a.H) a.out[(r * a.H + head) * kHeadDim + d] = (uint16_t)f2bf(v);
        }
      }
    }
  } else {
    const int64_t base = (r * a.nsplit + split) * a.H;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const int d = 128 * w + 16 * db + c16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int head = head0 + hb * 16 + 4 * g + i;
          if (head < a.H) a.part_o[(base + head) * kHeadDim + d] = (uint16_t)f2bf(o[hb][db][i]);
        }
      }
    if (w < HB && g == 0) {
      const int head = head0 + w * 16 + c16;
      if (head < a.H) {
        a.part_ml[(base + head) * 2 + 0] = m_run;
        a.part_ml[(base + head) * 2 + 1] = l_run;
      }
    }
  }
}

// Merge split-K partials with the sink; one workgroup of 128 threads per (query, head).
__global__ void __launch_bounds__(128)
merge_kernel(const uint16_t* __restrict__ part_o, const float* __restrict__ part_ml, int nsplit, int H,
             const float* __restrict__ sink, const int64_t* __restrict__ q_pos, int64_t rope_offset,
             RopeFreq rf, uint16_t* __restrict__ out) {
  const int64_t r = blockIdx.x;
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const float z = sink[h] * kLog2e;
  float M = z;
#pragma unroll 8
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, part_ml[((r * nsplit + s) * H + h) * 2]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float L = 0.f;
  if (M != -INFINITY) {
    L = exp2f(z - M);
#pragma unroll 8
    for (int s = 0; s < nsplit; ++s) {
      const int64_t base = (r * nsplit + s) * H + h;
      const float ms = part_ml[base * 2], ls = part_ml[base * 2 + 1];
      const float f = exp2f(ms - M);
      L += f * ls;
      const uint2 v = *reinterpret_cast<const uint2*>(part_o + base * kHeadDim + 4 * tid);
      acc.x += f * bf2f_lo(v.x); acc.y += f * bf2f_hi(v.x); acc.z += f * bf2f_lo(v.y); acc.w += f * bf2f_hi(v.y);
    }
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  float y0 = acc.x * inv, y1 = acc.y * inv, y2 = acc.z * inv, y3 = acc.w * inv;
  const int d0 = 4 * tid;
  if (d0 >= kRopeStart) {
    const double pos = (double)(q_pos[r] + rope_offset);
    float c, s;
    rope_cs(pos, rf.inv[(d0 - kRopeStart) / 2], &c, &s);
    const float r0 = y0 * c + y1 * s, r1 = -y0 * s + y1 * c;
    rope_cs(pos, rf.inv[(d0 - kRopeStart) / 2 + 1], &c, &s);
    const float r2 = y2 * c + y3 * s, r3 = -y2 * s + y3 * c;
    y0 = r0; y1 = r1; y2 = r2; y3 = r3;
  }
  uint2 o;
  o.x = pack_bf2(y0, y1);
  o.y = pack_bf2(y2, y3);
  *reinterpret_cast<uint2*>(out + (r * H + h) * kHeadDim + d0) = o;
}

inline size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

// 16-head blocks per workgroup (at most 2: 32 heads keep the tile loop within the register file)
// and the number of head-group workgroups per key split.
int head_blocks(int H) { return H <= 16 ? 1 : 2; }
int head_groups(int H) { return (H + 16 * head_blocks(H) - 1) / (16 * head_blocks(H)); }

// Keys per split: about one workgroup per CU (256) with at least 2 tiles (64 keys) each; every split
// adds a 64 KiB partial (bf16 O of 64 heads) that the merge reads back, so splits are kept few.
int keys_per_split(int R, int64_t max_keys) {
  const int64_t tiles = (max_keys + kTile - 1) / kTile;
  if (tiles <= 0) return kTile;
  int64_t want_splits = (256 + R - 1) / R;
  if (want_splits < 1) want_splits = 1;
  int64_t tps = (tiles + want_splits - 1) / want_splits;
  if (tps < 2) tps = 2;
  if (tps > tiles) tps = tiles;
  if (tps > kMaxSplitKeys / kTile) tps = kMaxSplitKeys / kTile;
  return (int)(tps * kTile);
}

}  // namespace

size_t attend_workspace(int B, int Tq, int H, int64_t max_keys) {
  const int R = B * Tq;
  const int kps = keys_per_split(R * head_groups(H), max_keys);
  const int64_t nsplit = max_keys > 0 ? (max_keys + kps - 1) / kps : 1;
  if (nsplit <= 1) return 256;
  return al256((size_t)R * nsplit * H * kHeadDim * 2) + al256((size_t)R * nsplit * H * 2 * 4);
}

int launch_attend(const AttendArgs& x, int64_t max_keys, hipStream_t st) {
  const int R = x.B * x.Tq;
  AttnK a;
  a.q = x.q; a.gamma_q = x.gamma_q; a.kv = x.kv; a.kv_ld = x.kv_ld; a.topk = x.topk; a.k = x.k;
  a.n_cap = x.n_cap; a.m = x.m; a.win = x.win; a.win_ld = x.win_ld; a.ring_cap = x.ring_cap;
  a.window = x.window; a.sink = x.sink; a.q_pos = x.q_pos; a.rope_offset = x.rope_offset;
  a.Tq = x.Tq; a.H = x.H; a.scale_log2 = x.scale * kLog2e; a.eps = x.eps; a.rf = rope_freq(x.theta);
  a.out = x.out;
  a.hgroups = head_groups(x.H);
  a.keys_per_split = keys_per_split(R * a.hgroups, max_keys);
  a.nsplit = max_keys > 0 ? (int)((max_keys + a.keys_per_split - 1) / a.keys_per_split) : 1;
  if (a.nsplit < 1) a.nsplit = 1;
  a.part_o = static_cast<uint16_t*>(x.ws);
  a.part_ml = reinterpret_cast<float*>(static_cast<char*>(x.ws) +
                                       al256((size_t)R * a.nsplit * x.H * kHeadDim * 2));
  dim3 grid((unsigned)(((a.nsplit + 7) / 8) * 8 * a.hgroups), (unsigned)R);
  if (head_blocks(x.H) == 1)
    LCS_LAUNCH("attend_kernel", attend_kernel<1>, grid, dim3(256), 0, st, a);
  else
    LCS_LAUNCH("attend_kernel", attend_kernel<2>, grid, dim3(256), 0, st, a);
  if (a.nsplit > 1) {
    LCS_LAUNCH("attend_merge_kernel", merge_kernel, dim3((unsigned)R, (unsigned)x.H), dim3(128), 0, st,
               a.part_o, a.part_ml, a.nsplit, x.H, x.sink, x.q_pos, x.rope_offset, a.rf, x.out);
  }
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // namespace lcs
