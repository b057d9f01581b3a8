// Position-free paged attention for gfx950: pic_attn_decode, pic_attn_prefill.
//
// What is computed (MiniPIC §2.1, score equation): for query row t of a
// request and each of its key slots j,
//     score(t, j) = (R_t q_t)^T (R_pi(j) k~_j) / sqrt(d)
// where k~_j is the UNROTATED key stored in a shared physical block, pi(j) is
// the key's logical position in this request, and R_p is the rotary rotation
// (rotate-half pairing, theta_i = base^(-2i/d), read from the cos/sin table).
// Softmax over the visible slots, then the weighted sum of the (unrotated)
// values.  Doing the rotation here instead of in the cache is algebraically
// the same as re-rotating the cache hit, without writing the shared block
// (MiniPIC §2.1, Implementation bullet).
//
// Formulation on the matrix cores (per kv head g and group of q heads):
//     S^T = K_rot * Q_rot^T      A = rotated keys (16 keys x d), B = queries
//     O^T += V^T * P^T           A = values transposed (d x keys), B = probs
// Keys are the M dimension of the score tile, so the score accumulator lands
// in exactly the register layout the PV product wants for its B operand (no
// shuffles), and V^T is read straight from the pool because the pool stores
// V transposed inside each block.  The rotation pairs element i with i + d/2;
// in this operand layout both halves of a pair sit in the same lane, so the
// rotation is a handful of FMAs on registers right after the load.
//
// Decode (one query row per request, memory bound): one wave per
// (request, kv head, key chunk), the G query heads of the kv head are the
// columns of the tile; K, V and the table row are read from global memory.
// Chunks of one request are merged in the same kernel: each chunk writes its
// normalised partial output and (max, sum) to the workspace, and the last
// workgroup of a (request, head group) to arrive merges them.
//
// Prefill (q_len > 1, MFMA bound): one workgroup per (request, kv head,
// 128 query rows); the rows are (token, q head of the group) pairs, 32 per
// wave.  Each 32-key step is gathered from the paged pool once per
// workgroup, rotated while it is written to LDS as the MFMA operand, and
// shared by the four waves; V^T is staged in LDS next to it.  Online softmax
// keeps one running max/sum per row.
#include <hip/hip_runtime.h>
#include <math.h>

#include <type_traits>

#include "pic.h"
#include "pic_common.hpp"
#include "pic_device.hpp"
#include "pic_host.hpp"

namespace pic {

struct AttnArgs {
  const void* q;
  const int32_t* cu_q;  // null for the decode-only kernel: row r is request r
  const int32_t* q_pos;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_table;
  long long bt_stride;
  const int32_t* seq_lens;
  const int32_t* cu_k;
  const int32_t* k_pos;
  const float* cos_tab;
  const float* sin_tab;
  int max_pos;
  int num_reqs;
  int hq;
  int hkv;
  int group;
  int num_blocks;
  int max_seq_len;
  int s_max;
  int nhg;
  float scale_log2;  // log2(e) / sqrt(d): scores are kept in base-2 units
  void* out;
  float2* ws_ml;
  float* ws_o;
  const int4* items;
  const int* nitems;
};

// seq_len of request r, clamped to what the grid, the workspace and the block
// table were sized for (a violated precondition gives wrong numbers, never an
// out-of-bounds access).
__device__ __forceinline__ int seq_len_of(const AttnArgs& a, int r) {
  const long long cap = min((long long)a.max_seq_len, a.bt_stride * kBlockSize);
  return (int)min((long long)a.seq_lens[r], cap);
}

// ---------------------------------------------------------------------------
// rotation helpers
// ---------------------------------------------------------------------------

// cos/sin of the pairs a lane owns: pair index c*KCH + grp*KPL + e for the
// first-half chunks c < NH, at table row `pos`.
template <typename T, int D>
__device__ __forceinline__ void load_trig(const AttnArgs& a, int pos, int grp, float* cs,
                                          float* sn) {
  using C = Cfg<T, D>;
  const float* crow = a.cos_tab + (size_t)pos * (D / 2) + grp * C::KPL;
  const float* srow = a.sin_tab + (size_t)pos * (D / 2) + grp * C::KPL;
#pragma unroll
  for (int c = 0; c < C::NH; ++c) {
    const typename Run<float, C::KPL>::V cv = Run<float, C::KPL>::load(crow + c * C::KCH);
    const typename Run<float, C::KPL>::V sv = Run<float, C::KPL>::load(srow + c * C::KCH);
#pragma unroll
    for (int e = 0; e < C::KPL; ++e) {
      cs[c * C::KPL + e] = elem<float, C::KPL>(cv, e);
      sn[c * C::KPL + e] = elem<float, C::KPL>(sv, e);
    }
  }
}

// x[c] and x[c + NH] hold the two halves of the same pairs: rotate in place.
template <typename T, int D>
__device__ __forceinline__ void rotate_ops(OpT<T>* x, const float* cs, const float* sn) {
  using C = Cfg<T, D>;
  using M = Mma<T>;
#pragma unroll
  for (int c = 0; c < C::NH; ++c) {
    float lo[C::KPL], hi[C::KPL];
#pragma unroll
    for (int e = 0; e < C::KPL; ++e) {
      const float a = M::get(x[c], e);
      const float b = M::get(x[c + C::NH], e);
      const float co = cs[c * C::KPL + e], si = sn[c * C::KPL + e];
      lo[e] = a * co - b * si;
      hi[e] = b * co + a * si;
    }
    x[c] = M::pack(lo);
    x[c + C::NH] = M::pack(hi);
  }
}

// Same rotation with the cos/sin values read from an LDS table row, one
// chunk at a time (cs/sn point at the lane's first pair of the row).
template <typename T, int D>
__device__ __forceinline__ void rotate_from_lds(OpT<T>* x, const float* cs, const float* sn) {
  using C = Cfg<T, D>;
  using M = Mma<T>;
  typedef Run<float, C::KPL> RF;
#pragma unroll
  for (int c = 0; c < C::NH; ++c) {
    const typename RF::V cv = RF::load(cs + c * C::KCH);
    const typename RF::V sv = RF::load(sn + c * C::KCH);
    float lo[C::KPL], hi[C::KPL];
#pragma unroll
    for (int e = 0; e < C::KPL; ++e) {
      const float a = M::get(x[c], e);
      const float b = M::get(x[c + C::NH], e);
      const float co = elem<float, C::KPL>(cv, e), si = elem<float, C::KPL>(sv, e);
      lo[e] = a * co - b * si;
      hi[e] = b * co + a * si;
    }
    x[c] = M::pack(lo);
    x[c + C::NH] = M::pack(hi);
  }
}

// Rotated query operand for one column: q row `qrow`, q head `head`.
template <typename T, int D>
__device__ __forceinline__ void load_query(const AttnArgs& a, long long qrow, int head, int pos,
                                           bool valid, int grp, OpT<T>* qop) {
  using C = Cfg<T, D>;
  using M = Mma<T>;
  const T* qp = (const T*)a.q + ((size_t)qrow * a.hq + head) * D + grp * C::KPL;
#pragma unroll
  for (int c = 0; c < C::NC; ++c) qop[c] = M::load(qp + c * C::KCH);
  float cs[C::NH * C::KPL], sn[C::NH * C::KPL];
  load_trig<T, D>(a, clampi(pos, 0, a.max_pos - 1), grp, cs, sn);
  rotate_ops<T, D>(qop, cs, sn);
  if (!valid) {
#pragma unroll
    for (int c = 0; c < C::NC; ++c) qop[c] = M::zero();
  }
}

// ---------------------------------------------------------------------------
// online softmax on one 16-column score tile set
// ---------------------------------------------------------------------------

// s[t][i]: masked scores (base-2 units, -inf where masked) of keys
// key_of(t, grp*4+i) for this lane's column.  Keeps a running base m per
// column (identical in the column's four lanes) and a lane-partial sum l,
// and overwrites s with 2^(s - m).  The base is only raised (and acc, l
// rescaled) when some column's new maximum exceeds it by more than
// kRescaleSlack, so most steps skip the rescale; the probabilities stay
// <= 2^kRescaleSlack and the final o = acc / l is unchanged.
constexpr float kRescaleSlack = 8.0f;

template <int NT, int ND>
__device__ __forceinline__ void softmax_step(f32x4 (&s)[NT], f32x4 (&acc)[ND], float& m,
                                             float& l) {
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[t][i]);
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  if (__any(mx > m + kRescaleSlack)) {
    const float m_new = fmaxf(m, mx);
    const float alpha = m_new == -INFINITY ? 1.0f : fast_exp2(m - m_new);
    l *= alpha;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) acc[dt] *= alpha;
    m = m_new;
  }
  const float base = (m == -INFINITY) ? 0.0f : m;
  float psum = 0.0f;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = fast_exp2(s[t][i] - base);
      s[t][i] = p;
      psum += p;
    }
  l += psum;
}

// B operand of PV MFMA number mi: probabilities of keys grp*4*NT + mi*KPL + e.
template <typename T, int D>
__device__ __forceinline__ typename Mma<T>::Op pack_probs(const f32x4 (&s)[Cfg<T, D>::NT],
                                                          int mi) {
  using C = Cfg<T, D>;
  float p[C::KPL];
#pragma unroll
  for (int e = 0; e < C::KPL; ++e) {
    const int idx = mi * C::KPL + e;
    p[e] = s[idx / 4][idx % 4];
  }
  return Mma<T>::pack(p);
}

__device__ __forceinline__ float col_sum(float l) {
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  return l;
}

template <typename T>
__device__ __forceinline__ void store4(T* p, f32x4 v, float scale) {
  if constexpr (sizeof(T) == 2) {
    vec<bf16, 4> o;
    o[0] = (bf16)(v[0] * scale);
    o[1] = (bf16)(v[1] * scale);
    o[2] = (bf16)(v[2] * scale);
    o[3] = (bf16)(v[3] * scale);
    *reinterpret_cast<vec<bf16, 4>*>(p) = o;
  } else {
    *reinterpret_cast<f32x4*>(p) = v * scale;
  }
}

// ---------------------------------------------------------------------------
// decode: one wave = (request r, kv head g, keys [k0, k1)), q row qrow
// ---------------------------------------------------------------------------

// Upper bound of split_len: a chunk never exceeds 1.5x the split target
// (rounded up to whole steps).
constexpr int kMaxChunk = kSplitTarget + kSplitTarget / 2 + 32;

// LDS of a decode workgroup: the chunk's key positions and block ids, and
// the cos/sin rows of two steps (one row per key of the step, padded so the
// 16 rows one read instruction touches fall in different banks).
template <typename T, int D>
struct DecodeSmem {
  static constexpr int KSTEP = Cfg<T, D>::KSTEP;
  static constexpr int TLD = D / 2 + 4;
  float cs[2][KSTEP][TLD];
  float sn[2][KSTEP][TLD];
  int pos[kMaxChunk];
  int blk[kMaxChunk / kBlockSize + 2];
};

// One decode work item: request r, key chunk s, kv heads hg*4 .. hg*4+3 (one
// per wave).  All four waves walk the same keys: each step's cos/sin rows are
// fetched once per workgroup and shared through LDS, while every wave reads
// its own head's K rows and V runs from the pools into registers.  NB steps
// of loads are kept in flight (a ring of NB register buffers): the loads of
// step j+NB are issued as soon as step j has consumed its buffer.  The
// chunk's block ids and key positions are staged in LDS first, so no
// address lookup ever waits behind the data loads.  With one chunk the wave
// writes the output row; otherwise it writes a normalised partial and
// (max, sum) that combine_kernel merges.  Uniform across the workgroup.
template <typename T, int D, int NB>
__device__ void decode_item(const AttnArgs& a, int r, int hg, int s, long long qrow,
                            unsigned char* smem_raw) {
  using C = Cfg<T, D>;
  using M = Mma<T>;
  typedef typename M::Op Op;
  DecodeSmem<T, D>& sm = *reinterpret_cast<DecodeSmem<T, D>*>(smem_raw);
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int row16 = lane & 15;
  const int grp = lane >> 4;
  const int g = hg * kWaves + wave;
  const bool active = g < a.hkv;
  const int ga = active ? g : 0;  // a valid head for the loads of an idle wave
  const int G = a.group;
  const int L = seq_len_of(a, r);
  const int S = num_splits(L, C::KSTEP);
  if (s >= S) return;
  if (L <= 0) {  // empty context: zero output
    if (active) {
      T* out = (T*)a.out + ((size_t)qrow * a.hq + g * G) * D;
      for (int e = lane; e < G * D; e += 64) out[e] = (T)0.0f;
    }
    return;
  }
  const int chunk = split_len(L, C::KSTEP);
  const int k0 = s * chunk;
  const int k1 = min(L, k0 + chunk);
  const int nsteps = cdiv(k1 - k0, C::KSTEP);

  // chunk metadata -> LDS: positions of keys k0.., block ids of blocks k0/16..
  {
    const int32_t* bt = a.block_table + (size_t)r * a.bt_stride;
    const int32_t* kp = a.k_pos + a.cu_k[r];
    const int nk = nsteps * C::KSTEP;
    for (int j = tid; j < nk; j += kThreads)
      sm.pos[j] = clampi(kp[min(k0 + j, L - 1)], 0, a.max_pos - 1);
    const int nbk = nk / kBlockSize;
    for (int j = tid; j < nbk; j += kThreads)
      sm.blk[j] = clampi(bt[min((k0 >> 4) + j, (L - 1) >> 4)], 0, a.num_blocks - 1);
  }

  Op qop[C::NC];
  const bool qvalid = row16 < G;
  load_query<T, D>(a, qrow, ga * G + (qvalid ? row16 : 0), a.q_pos[qrow], qvalid, grp, qop);
  __syncthreads();

  const T* kpool = (const T*)a.k_pool;
  const T* vpool = (const T*)a.v_pool;
  const size_t head_k = (size_t)ga * kBlockSize * D;
  const size_t head_v = (size_t)ga * D * kBlockSize;
  const size_t blk_stride = (size_t)a.hkv * kBlockSize * D;
  // this lane's key block inside a step (the K row of its A-operand row, the
  // V run of its lane group) for steps that span two blocks (bf16)
  const int kblk_sel = (key_of<C::NT>(0, row16) >= kBlockSize) ? 1 : 0;
  const int vblk_sel = (grp * 4 * C::NT >= kBlockSize) ? 1 : 0;
  const int vkey_off = (grp * 4 * C::NT) & 15;

  // table staging: thread -> (key of the step, TPT consecutive pairs)
  constexpr int TPT = C::KSTEP * (D / 2) / kThreads;
  constexpr int TPK = (D / 2) / TPT;
  typedef Run<float, TPT> RF;
  const int skey = tid / TPK;
  const int spart = (tid % TPK) * TPT;

  struct Group {
    Op k[C::NT][C::NC];
    Op v[C::NPV][C::ND];
    typename RF::V c, sn;
  };
  Group grpbuf[NB];

  // issue every load of step j (relative to k0) into a register group
  auto issue = [&](int j, Group& gb) {
    const int kb = j * C::KSTEP;  // offset in the chunk
    const int b0 = sm.blk[kb >> 4];
    const int b1 = sm.blk[min((kb >> 4) + 1, nsteps * C::KSTEP / kBlockSize - 1)];
#pragma unroll
    for (int t = 0; t < C::NT; ++t) {
      const int kk = key_of<C::NT>(t, row16);
      const int blk = (kblk_sel ? b1 : b0);
      const T* krow = kpool + (size_t)blk * blk_stride + head_k +
                      (size_t)((kb + kk) & 15) * D + grp * C::KPL;
#pragma unroll
      for (int c = 0; c < C::NC; ++c) gb.k[t][c] = M::load(krow + c * C::KCH);
    }
#pragma unroll
    for (int mi = 0; mi < C::NPV; ++mi) {
      const int blk = (vblk_sel ? b1 : b0);
      const T* vrow = vpool + (size_t)blk * blk_stride + head_v + (size_t)row16 * kBlockSize +
                      ((vkey_off + mi * C::KPL) & 15);
#pragma unroll
      for (int dt = 0; dt < C::ND; ++dt) gb.v[mi][dt] = M::load(vrow + (size_t)dt * 16 * kBlockSize);
    }
    const size_t row = (size_t)sm.pos[kb + skey] * (D / 2) + spart;
    gb.c = RF::load(a.cos_tab + row);
    gb.sn = RF::load(a.sin_tab + row);
  };

  f32x4 acc[C::ND];
#pragma unroll
  for (int dt = 0; dt < C::ND; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;

#pragma unroll
  for (int b = 0; b < NB; ++b)
    if (b < nsteps) issue(b, grpbuf[b]);

  // step j with its loads in group gb; buf: LDS table slot
  auto step = [&](int j, Group& gb) {
    const int buf = j & 1;
    const int kb = k0 + j * C::KSTEP;  // absolute key index
    RF::store(&sm.cs[buf][skey][spart], gb.c);
    RF::store(&sm.sn[buf][skey][spart], gb.sn);
    __syncthreads();
    f32x4 sc[C::NT];
#pragma unroll
    for (int t = 0; t < C::NT; ++t) {
      const int krow = key_of<C::NT>(t, row16);
      rotate_from_lds<T, D>(gb.k[t], &sm.cs[buf][krow][grp * C::KPL],
                            &sm.sn[buf][krow][grp * C::KPL]);
      sc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < C::NC; ++c) sc[t] = M::run(gb.k[t][c], qop[c], sc[t]);
    }
#pragma unroll
    for (int t = 0; t < C::NT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kb + key_of<C::NT>(t, grp * 4 + i);
        sc[t][i] = key < k1 ? sc[t][i] * a.scale_log2 : -INFINITY;
      }
    softmax_step<C::NT, C::ND>(sc, acc, m_run, l_run);
    // slots at or beyond L hold no data: clear those V elements (bit mask,
    // all ones except in a request's last step)
#pragma unroll
    for (int mi = 0; mi < C::NPV; ++mi) {
      const int vkey = kb + grp * 4 * C::NT + mi * C::KPL;
      const int nvalid = L - vkey;
      if (nvalid < C::KPL) {
#pragma unroll
        for (int dt = 0; dt < C::ND; ++dt)
#pragma unroll
          for (int e = 0; e < C::KPL; ++e)
            if (e >= nvalid) M::set(gb.v[mi][dt], e, 0.0f);
      }
    }
#pragma unroll
    for (int mi = 0; mi < C::NPV; ++mi) {
      const Op p = pack_probs<T, D>(sc, mi);
#pragma unroll
      for (int dt = 0; dt < C::ND; ++dt) acc[dt] = M::run(gb.v[mi][dt], p, acc[dt]);
    }
    if (j + NB < nsteps) issue(j + NB, gb);
  };

  for (int j0 = 0; j0 < nsteps; j0 += NB) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
      if (j0 + b < nsteps) step(j0 + b, grpbuf[b]);
  }

  const float l_tot = col_sum(l_run);
  if (!active || row16 >= G) return;
  const float inv = 1.0f / l_tot;
  if (S == 1) {
    T* out = (T*)a.out + ((size_t)qrow * a.hq + g * G + row16) * D + grp * 4;
#pragma unroll
    for (int dt = 0; dt < C::ND; ++dt) store4<T>(out + dt * 16, acc[dt], inv);
    return;
  }
  const size_t pidx = (((size_t)r * a.hkv + g) * a.s_max + s) * G + row16;
  float* po = a.ws_o + pidx * D + grp * 4;
#pragma unroll
  for (int dt = 0; dt < C::ND; ++dt) *reinterpret_cast<f32x4*>(po + dt * 16) = acc[dt] * inv;
  if (grp == 0) a.ws_ml[pidx] = make_float2(m_run, l_tot);
}

// Merge the chunk partials of every multi-chunk q_len == 1 request:
// o = sum_s w_s o_s / sum_s w_s with w_s = l_s 2^(m_s - max m).  One
// workgroup per (request, kv head); threads take (column, 8 consecutive d)
// pairs, and threads beyond those pairs take every SG-th chunk in parallel.
template <typename T, int D>
__global__ void __launch_bounds__(kThreads) combine_kernel(AttnArgs a) {
  constexpr int EPT = 8;
  __shared__ __attribute__((aligned(16))) float gm[kThreads * EPT];
  __shared__ float2 gml[kThreads];
  const int tid = threadIdx.x;
  const int r = blockIdx.x / a.hkv;
  const int g = blockIdx.x % a.hkv;
  if (a.cu_q && a.cu_q[r + 1] - a.cu_q[r] != 1) return;
  const long long qrow = a.cu_q ? (long long)a.cu_q[r] : (long long)r;
  const int L = seq_len_of(a, r);
  const int S = num_splits(L, Cfg<T, D>::KSTEP);
  if (L <= 0 || S <= 1) return;
  const int G = a.group;
  const int pairs = G * (D / EPT);
  const int SG = max(1, kThreads / pairs);
  const int sg = tid / pairs;
  const int pc = tid % pairs;
  const int col = pc / (D / EPT);
  const int d0 = (pc % (D / EPT)) * EPT;
  const size_t pbase = ((size_t)r * a.hkv + g) * a.s_max;
  float pm = -INFINITY, pl = 0.0f;
  float po[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) po[e] = 0.0f;
  if (sg < SG) {
#pragma unroll 4
    for (int ss = sg; ss < S; ss += SG) {
      const float2 ml = a.ws_ml[(pbase + ss) * G + col];
      const float* src = a.ws_o + ((pbase + ss) * G + col) * D + d0;
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(src);
      const f32x4 x1 = *reinterpret_cast<const f32x4*>(src + 4);
      const float mn = fmaxf(pm, ml.x);
      const float a0 = fast_exp2(pm - mn), a1 = ml.y * fast_exp2(ml.x - mn);
      pl = pl * a0 + a1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        po[e] = po[e] * a0 + a1 * x0[e];
        po[e + 4] = po[e + 4] * a0 + a1 * x1[e];
      }
      pm = mn;
    }
#pragma unroll
    for (int e = 0; e < EPT; ++e) gm[tid * EPT + e] = po[e];
    gml[tid] = make_float2(pm, pl);
  }
  __syncthreads();
  if (tid >= pairs) return;
  float mm = -INFINITY;
  for (int j = 0; j < SG; ++j) mm = fmaxf(mm, gml[j * pairs + tid].x);
  float ll = 0.0f, oo[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) oo[e] = 0.0f;
  for (int j = 0; j < SG; ++j) {
    const float2 ml = gml[j * pairs + tid];
    if (ml.y == 0.0f) continue;  // a chunk group with no chunk
    const float w = fast_exp2(ml.x - mm);
    ll += w * ml.y;
#pragma unroll
    for (int e = 0; e < EPT; ++e) oo[e] += w * gm[(j * pairs + tid) * EPT + e];
  }
  const float inv = 1.0f / ll;
  T* dst = (T*)a.out + ((size_t)qrow * a.hq + g * G + col) * D + d0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) dst[e] = (T)(oo[e] * inv);
}

// ---------------------------------------------------------------------------
// prefill tile: request r, kv head g, query rows [tile*128, tile*128+128)
// ---------------------------------------------------------------------------

template <typename T, int D>
struct PrefillSmem {
  using C = Cfg<T, D>;
  static constexpr int KLD = D + C::PAD;            // K row stride (elements)
  static constexpr int VLD = C::KSTEP + C::PAD;     // V^T row stride (elements)
  static constexpr int BYTES = (C::KSTEP * KLD + D * VLD) * (int)sizeof(T);
};

template <typename T, int D>
__device__ void prefill_tile(const AttnArgs& a, int r, int g, int tile, unsigned char* smem) {
  using C = Cfg<T, D>;
  using M = Mma<T>;
  using SM = PrefillSmem<T, D>;
  typedef typename M::Op Op;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int row16 = lane & 15;
  const int grp = lane >> 4;
  const int G = a.group;
  const int q0 = a.cu_q[r];
  const int ql = a.cu_q[r + 1] - q0;
  const int L = seq_len_of(a, r);
  const int nrows = ql * G;
  const int trow0 = tile * kPrefillRows;
  const int last_tok = min((trow0 + kPrefillRows - 1) / G, ql - 1);
  const int kend = min(L, L - ql + last_tok + 1);  // slots any row of the tile sees

  Op qop[2][C::NC];
  int lim[2];      // last visible slot of the column, -1 for padding columns
  int tok_of[2], head_of[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = trow0 + wave * 32 + j * 16 + row16;
    const bool valid = n < nrows;
    const int nn = valid ? n : 0;
    tok_of[j] = nn / G;
    head_of[j] = nn % G;
    lim[j] = valid ? L - ql + tok_of[j] : -1;
    load_query<T, D>(a, (long long)q0 + tok_of[j], g * G + head_of[j], a.q_pos[q0 + tok_of[j]],
                     valid, grp, qop[j]);
  }

  T* Ks = reinterpret_cast<T*>(smem);
  T* Vs = Ks + C::KSTEP * SM::KLD;
  const int32_t* bt = a.block_table + (size_t)r * a.bt_stride;
  const int32_t* kp = a.k_pos + a.cu_k[r];
  const T* kpool = (const T*)a.k_pool;
  const T* vpool = (const T*)a.v_pool;
  const int nb_max = a.num_blocks - 1;
  const int pmax = a.max_pos - 1;

  f32x4 acc[2][C::ND];
  float m_run[2], l_run[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int dt = 0; dt < C::ND; ++dt) acc[j][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[j] = -INFINITY;
    l_run[j] = 0.0f;
  }

  // cooperative staging shapes
  constexpr int PPT = C::KSTEP * (D / 2) / kThreads;  // rotation pairs per thread
  constexpr int TPK = (D / 2) / PPT;                  // threads per key
  constexpr int EPT = C::KSTEP * D / kThreads;        // V elements per thread
  constexpr int TPR = C::KSTEP / EPT;                 // threads per V^T row
  static_assert(PPT >= 1 && EPT >= 1 && EPT <= kBlockSize, "staging shape");

  for (int kb = 0; kb < kend; kb += C::KSTEP) {
    {  // rotated K rows -> LDS
      const int key = threadIdx.x / TPK;
      const int i0 = (threadIdx.x % TPK) * PPT;
      const int kc = min(kb + key, L - 1);
      const int blk = clampi(bt[kc >> 4], 0, nb_max);
      const int pos = clampi(kp[kc], 0, pmax);
      const T* src = kpool + (((size_t)blk * a.hkv + g) * kBlockSize + (kc & 15)) * D + i0;
      typedef Run<T, PPT> RT;
      typedef Run<float, PPT> RF;
      typename RT::V lo = RT::load(src), hi = RT::load(src + D / 2);
      const typename RF::V cv = RF::load(a.cos_tab + (size_t)pos * (D / 2) + i0);
      const typename RF::V sv = RF::load(a.sin_tab + (size_t)pos * (D / 2) + i0);
#pragma unroll
      for (int e = 0; e < PPT; ++e) {
        const float x = elem<T, PPT>(lo, e), y = elem<T, PPT>(hi, e);
        const float c = elem<float, PPT>(cv, e), sn = elem<float, PPT>(sv, e);
        set_elem<T, PPT>(lo, e, x * c - y * sn);
        set_elem<T, PPT>(hi, e, y * c + x * sn);
      }
      RT::store(Ks + key * SM::KLD + i0, lo);
      RT::store(Ks + key * SM::KLD + D / 2 + i0, hi);
    }
    {  // V^T rows -> LDS (keys at or beyond L are zeroed)
      const int d = threadIdx.x / TPR;
      const int kr0 = (threadIdx.x % TPR) * EPT;
      const int vk = kb + kr0;
      const int vkc = min(vk, L - 1);
      const int blk = clampi(bt[vkc >> 4], 0, nb_max);
      const T* src = vpool + (((size_t)blk * a.hkv + g) * D + d) * kBlockSize + (vk & 15);
      T* dst = Vs + d * SM::VLD + kr0;
      constexpr int VEC = 16 / (int)sizeof(T);
      constexpr int NV = EPT >= VEC ? EPT / VEC : 1;
      constexpr int W = EPT >= VEC ? VEC : EPT;
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        typename Run<T, W>::V x = Run<T, W>::load(src + u * W);
        if (vk + (u + 1) * W > L) {
#pragma unroll
          for (int e = 0; e < W; ++e)
            if (vk + u * W + e >= L) set_elem<T, W>(x, e, 0.0f);
        }
        Run<T, W>::store(dst + u * W, x);
      }
    }
    __syncthreads();

    f32x4 s[2][C::NT];
#pragma unroll
    for (int t = 0; t < C::NT; ++t) {
      const T* kr = Ks + key_of<C::NT>(t, row16) * SM::KLD + grp * C::KPL;
      Op kop[C::NC];
#pragma unroll
      for (int c = 0; c < C::NC; ++c) kop[c] = M::load(kr + c * C::KCH);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        s[j][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < C::NC; ++c) s[j][t] = M::run(kop[c], qop[j][c], s[j][t]);
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int t = 0; t < C::NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kb + key_of<C::NT>(t, grp * 4 + i);
          s[j][t][i] = key <= lim[j] ? s[j][t][i] * a.scale_log2 : -INFINITY;
        }
      softmax_step<C::NT, C::ND>(s[j], acc[j], m_run[j], l_run[j]);
    }
#pragma unroll
    for (int mi = 0; mi < C::NPV; ++mi) {
      Op p[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) p[j] = pack_probs<T, D>(s[j], mi);
      const T* vr = Vs + row16 * SM::VLD + grp * 4 * C::NT + mi * C::KPL;
#pragma unroll
      for (int dt = 0; dt < C::ND; ++dt) {
        const Op v = M::load(vr + dt * 16 * SM::VLD);
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[j][dt] = M::run(v, p[j], acc[j][dt]);
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float l_tot = col_sum(l_run[j]);
    if (lim[j] >= 0) {
      T* out = (T*)a.out + (((size_t)q0 + tok_of[j]) * a.hq + g * G + head_of[j]) * D + grp * 4;
      const float inv = 1.0f / l_tot;
#pragma unroll
      for (int dt = 0; dt < C::ND; ++dt) store4<T>(out + dt * 16, acc[j][dt], inv);
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 prefill tile on 32x32x16 MFMAs: request r, kv head g, query rows
// [tile*ROWS, tile*ROWS + ROWS), ROWS = 4 waves x 32 x NCB
// ---------------------------------------------------------------------------

template <int D, int NCB>
struct Pf {
  static constexpr int KSTEP = 64;                 // keys per step
  static constexpr int ROWS = kWaves * 32 * NCB;   // query rows per tile
  static constexpr int NCH = D / 16;               // 16-wide d chunks (MFMA K)
  static constexpr int NHC = NCH / 2;              // chunks of the first half of d
  static constexpr int NDB = D / 32;               // 32-row d blocks of O^T
  static constexpr int KLD = D + 8;                // LDS K row stride (bf16)
  static constexpr int VLD = KSTEP + 8;            // LDS V^T row stride (bf16)
  static constexpr int STAGE = KSTEP * KLD + D * VLD;  // bf16 elements per LDS stage
  static constexpr int BYTES = 2 * STAGE * 2;      // two stages
  static constexpr int KPT = KSTEP * (D / 2) / kThreads;  // rotation pairs per thread
  static constexpr int KTPK = (D / 2) / KPT;              // threads per key
  static constexpr int VPT = KSTEP * D / kThreads;        // V elements per thread
  static constexpr int VTPR = KSTEP / VPT;                // threads per V^T row
  static_assert(VPT % kBlockSize == 0, "a thread stages whole 16-key V runs");
};

// One prefill tile, bf16.  Each 64-key step is gathered from the paged pools
// once per workgroup: every thread loads its share of K rows, cos/sin rows and
// V^T runs into registers one step ahead (the loads fly while the previous
// step computes), then rotates its K pairs and writes K and V^T into the
// other half of a double-buffered LDS stage.  One barrier per step.  Each
// wave owns 32*NCB query rows (the B operand, rotated once) and runs
// 2*NCB*NCH score MFMAs and 4*NCB*NDB PV MFMAs per step.  Steps that lie
// wholly below the causal diagonal skip the mask.
template <int D, int NCB>
__device__ void prefill_tile_bf16(const AttnArgs& a, int r, int g, int tile,
                                  unsigned char* smem) {
  using P = Pf<D, NCB>;
  typedef Mma32::Op Op;
  typedef Mma32::Acc Acc;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;
  const int hh = lane >> 5;
  const int G = a.group;
  const int q0 = a.cu_q[r];
  const int ql = a.cu_q[r + 1] - q0;
  const int L = seq_len_of(a, r);
  const int nrows = ql * G;
  const int trow0 = tile * P::ROWS;
  const int first_tok = trow0 / G;
  const int last_tok = min((trow0 + P::ROWS - 1) / G, ql - 1);
  const int kend = min(L, L - ql + last_tok + 1);  // slots any row of the tile sees
  const int kfull = max(0, L - ql + first_tok + 1);  // slots every row of the tile sees
  const int nsteps = cdiv(kend, P::KSTEP);

  // rotated query operands (B of S^T = K Q^T), one per column block and d chunk
  Op qop[NCB][P::NCH];
  int lim[NCB], tok_of[NCB], head_of[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int n = trow0 + wave * 32 * NCB + cb * 32 + col;
    const bool valid = n < nrows;
    const int nn = valid ? n : 0;
    tok_of[cb] = nn / G;
    head_of[cb] = nn % G;
    lim[cb] = valid ? L - ql + tok_of[cb] : -1;
    const bf16* qp = (const bf16*)a.q + (((size_t)q0 + tok_of[cb]) * a.hq + g * G + head_of[cb]) * D +
                     hh * 8;
    const int pos = clampi(a.q_pos[q0 + tok_of[cb]], 0, a.max_pos - 1);
    const float* cr = a.cos_tab + (size_t)pos * (D / 2) + hh * 8;
    const float* sr = a.sin_tab + (size_t)pos * (D / 2) + hh * 8;
#pragma unroll
    for (int c = 0; c < P::NCH; ++c) qop[cb][c] = *reinterpret_cast<const Op*>(qp + c * 16);
#pragma unroll
    for (int c = 0; c < P::NHC; ++c) {
      const vec<float, 8> cv = *reinterpret_cast<const vec<float, 8>*>(cr + c * 16);
      const vec<float, 8> sv = *reinterpret_cast<const vec<float, 8>*>(sr + c * 16);
      float lo[8], hi[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = (float)qop[cb][c][e], y = (float)qop[cb][c + P::NHC][e];
        lo[e] = x * cv[e] - y * sv[e];
        hi[e] = y * cv[e] + x * sv[e];
      }
      qop[cb][c] = Mma<bf16>::pack(lo);
      qop[cb][c + P::NHC] = Mma<bf16>::pack(hi);
    }
    if (!valid) {
#pragma unroll
      for (int c = 0; c < P::NCH; ++c) qop[cb][c] = Mma<bf16>::zero();
    }
  }

  bf16* stage0 = reinterpret_cast<bf16*>(smem);
  const int32_t* bt = a.block_table + (size_t)r * a.bt_stride;
  const int32_t* kp = a.k_pos + a.cu_k[r];
  const bf16* kpool = (const bf16*)a.k_pool;
  const bf16* vpool = (const bf16*)a.v_pool;
  const int nb_max = a.num_blocks - 1;
  const int pmax = a.max_pos - 1;
  const size_t blk_stride = (size_t)a.hkv * kBlockSize * D;

  // staging: thread -> (key, KPT pairs) for K and the table, (d row, VPT keys) for V
  const int skey = tid / P::KTPK;
  const int si0 = (tid % P::KTPK) * P::KPT;
  const int vd = tid / P::VTPR;
  const int vk0 = (tid % P::VTPR) * P::VPT;
  typedef vec<bf16, P::KPT> KV;
  typedef vec<float, P::KPT> TV;
  typedef vec<bf16, kBlockSize> VR;
  KV klo, khi;
  TV tc, ts;
  VR vr[P::VPT / kBlockSize];
  // addresses of a step (block ids, position): looked up one step before the
  // step's data loads are issued, so those never wait on the lookup
  struct StepMeta {
    int kblk, koff, pos;
    int vblk[P::VPT / kBlockSize];
  };
  auto load_meta = [&](int kb, StepMeta& sm_) {
    const int kc = min(kb + skey, L - 1);
    sm_.kblk = bt[kc >> 4];
    sm_.koff = kc & 15;
    sm_.pos = kp[kc];
#pragma unroll
    for (int u = 0; u < P::VPT / kBlockSize; ++u)
      sm_.vblk[u] = bt[min(kb + vk0 + u * kBlockSize, L - 1) >> 4];
  };
  auto load_step = [&](const StepMeta& sm_) {
    const int blk = clampi(sm_.kblk, 0, nb_max);
    const int pos = clampi(sm_.pos, 0, pmax);
    const bf16* src = kpool + blk * blk_stride + ((size_t)g * kBlockSize + sm_.koff) * D + si0;
    klo = *reinterpret_cast<const KV*>(src);
    khi = *reinterpret_cast<const KV*>(src + D / 2);
    tc = *reinterpret_cast<const TV*>(a.cos_tab + (size_t)pos * (D / 2) + si0);
    ts = *reinterpret_cast<const TV*>(a.sin_tab + (size_t)pos * (D / 2) + si0);
#pragma unroll
    for (int u = 0; u < P::VPT / kBlockSize; ++u) {
      const int vb = clampi(sm_.vblk[u], 0, nb_max);
      vr[u] = *reinterpret_cast<const VR*>(vpool + vb * blk_stride +
                                           ((size_t)g * D + vd) * kBlockSize);
    }
  };
  auto store_step = [&](int kb, bf16* st, auto tail_tag) {
    constexpr bool TAIL = decltype(tail_tag)::value;
    float lo[P::KPT], hi[P::KPT];
#pragma unroll
    for (int e = 0; e < P::KPT; ++e) {
      const float x = (float)klo[e], y = (float)khi[e];
      lo[e] = x * tc[e] - y * ts[e];
      hi[e] = y * tc[e] + x * ts[e];
    }
    bf16* kd = st + skey * P::KLD + si0;
#pragma unroll
    for (int e0 = 0; e0 < P::KPT; e0 += 8) {
      *reinterpret_cast<Op*>(kd + e0) = Mma<bf16>::pack(lo + e0);
      *reinterpret_cast<Op*>(kd + D / 2 + e0) = Mma<bf16>::pack(hi + e0);
    }
    bf16* vdst = st + P::KSTEP * P::KLD + vd * P::VLD + vk0;
#pragma unroll
    for (int u = 0; u < P::VPT / kBlockSize; ++u) {
      VR x = vr[u];
      if constexpr (TAIL) {  // slots at or beyond L hold no data
        const int key0 = kb + vk0 + u * kBlockSize;
#pragma unroll
        for (int e = 0; e < kBlockSize; ++e)
          if (key0 + e >= L) x[e] = (bf16)0.0f;
      }
      *reinterpret_cast<VR*>(vdst + u * kBlockSize) = x;
    }
  };

  Acc o[P::NDB][NCB];
  float m_run[NCB], l_run[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
    for (int db = 0; db < P::NDB; ++db) o[db][cb] = Acc{};
    m_run[cb] = -INFINITY;
    l_run[cb] = 0.0f;
  }

  // staging of step kb: only a step that reaches past L needs the V zeroing
  auto store_any = [&](int kb, bf16* st) {
    if (kb + P::KSTEP > L) store_step(kb, st, std::true_type{});
    else store_step(kb, st, std::false_type{});
  };
  StepMeta meta;  // addresses of the step after the one being loaded
  if (nsteps > 0) {
    load_meta(0, meta);
    load_step(meta);
    if (nsteps > 1) load_meta(P::KSTEP, meta);
    store_any(0, stage0);
  }
  __syncthreads();

  // steps wholly below the causal diagonal of every row skip the mask
  auto step = [&](int j, auto mask_tag) {
    constexpr bool MASKED = decltype(mask_tag)::value;
    const int kb = j * P::KSTEP;
    const bf16* st = stage0 + (j & 1) * P::STAGE;
    if (j + 1 < nsteps) {
      load_step(meta);
      if (j + 2 < nsteps) load_meta(kb + 2 * P::KSTEP, meta);
    }

    // S^T = K_rot Q_rot^T for the step's two 32-key blocks
    Acc sc[2][NCB];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) sc[kb2][cb] = Acc{};
      const bf16* krow = st + (kb2 * 32 + key32(col)) * P::KLD + hh * 8;
#pragma unroll
      for (int c = 0; c < P::NCH; ++c) {
        const Op ka = *reinterpret_cast<const Op*>(krow + c * 16);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) sc[kb2][cb] = Mma32::run(ka, qop[cb][c], sc[kb2][cb]);
      }
    }

    // causal mask (masked steps only), online softmax per column (scores kept
    // raw: the base-2 scale is folded into the exponent's FMA), probabilities
    // -> bf16 B operands
    Op pb[2][2][NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          if constexpr (MASKED) {
            const int key = kb + kb2 * 32 + key32(8 * (v >> 2) + 4 * hh + (v & 3));
            if (key > lim[cb]) sc[kb2][cb][v] = -INFINITY;
          }
          mx = fmaxf(mx, sc[kb2][cb][v]);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32)) * a.scale_log2;
      if (__any(mx > m_run[cb] + kRescaleSlack)) {
        const float m_new = fmaxf(m_run[cb], mx);
        const float alpha = m_new == -INFINITY ? 1.0f : fast_exp2(m_run[cb] - m_new);
        l_run[cb] *= alpha;
#pragma unroll
        for (int db = 0; db < P::NDB; ++db) o[db][cb] *= alpha;
        m_run[cb] = m_new;
      }
      const float nbase = m_run[cb] == -INFINITY ? 0.0f : -m_run[cb];
      float psum = 0.0f;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          float p[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            p[e] = fast_exp2(fmaf(sc[kb2][cb][8 * m + e], a.scale_log2, nbase));
            psum += p[e];
          }
          pb[kb2][m][cb] = Mma<bf16>::pack(p);
        }
      l_run[cb] += psum;
    }

    // O^T += V^T P^T
    const bf16* vs = st + P::KSTEP * P::KLD;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int db = 0; db < P::NDB; ++db) {
          const Op va = *reinterpret_cast<const Op*>(vs + (db * 32 + col) * P::VLD + kb2 * 32 +
                                                     16 * m + 8 * hh);
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) o[db][cb] = Mma32::run(va, pb[kb2][m][cb], o[db][cb]);
        }

    if (j + 1 < nsteps) store_any(kb + P::KSTEP, stage0 + ((j + 1) & 1) * P::STAGE);
    __syncthreads();
  };

  // the leading steps lie below every row's causal limit: no mask there
  const int jfull = min(nsteps, kfull / P::KSTEP);
  for (int j = 0; j < jfull; ++j) step(j, std::false_type{});
  for (int j = jfull; j < nsteps; ++j) step(j, std::true_type{});

#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const float l_tot = l_run[cb] + __shfl_xor(l_run[cb], 32);
    if (lim[cb] < 0) continue;
    const float inv = 1.0f / l_tot;
    bf16* out = (bf16*)a.out + (((size_t)q0 + tok_of[cb]) * a.hq + g * G + head_of[cb]) * D;
#pragma unroll
    for (int db = 0; db < P::NDB; ++db)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        vec<bf16, 4> w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = (bf16)(o[db][cb][4 * v4 + i] * inv);
        *reinterpret_cast<vec<bf16, 4>*>(out + db * 32 + 8 * v4 + 4 * hh) = w;
      }
  }
}

// ---------------------------------------------------------------------------
// kernels
// ---------------------------------------------------------------------------

// Workgroup b runs on XCD b % 8 (round-robin dispatch).  Give each XCD a
// contiguous range of logical items so items that share data (the same
// table rows, the same request's blocks) share that XCD's L2.
__device__ __forceinline__ long long xcd_logical(long long b, long long n) {
  const long long q = n / 8, rem = n % 8;
  const long long x = b % 8, k = b / 8;
  return x * q + min(x, rem) + k;
}
// Inverse of xcd_logical: dispatch position of logical item l.
__device__ __forceinline__ long long xcd_position(long long l, long long n) {
  const long long q = n / 8, rem = n % 8;
  long long x, k;
  if (l < rem * (q + 1)) {
    x = l / (q + 1);
    k = l % (q + 1);
  } else {
    x = rem + (l - rem * (q + 1)) / q;
    k = (l - rem * (q + 1)) % q;
  }
  return k * 8 + x;
}

// Steps of K/V loads each decode wave keeps in flight.  Measured on MI355X:
// one step at two waves per SIMD beats deeper rings at one wave per SIMD.
constexpr int kDecodeDepth = 1;

// Decode-only launch: logical item = (chunk s, request r, head group hg),
// head group fastest, then request: the workgroups that read the same table
// rows (the same key positions) run on one XCD and share its L2.
template <typename T, int D>
__global__ void __launch_bounds__(kThreads, 2) decode_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[sizeof(DecodeSmem<T, D>)];
  const long long n = (long long)gridDim.x;
  const long long l = xcd_logical(blockIdx.x, n);
  const int hg = (int)(l % a.nhg);
  const long long rs = l / a.nhg;
  const int r = (int)(rs % a.num_reqs);
  const int s = (int)(rs / a.num_reqs);
  decode_item<T, D, kDecodeDepth>(a, r, hg, s, r, smem);
}

// Column blocks (of 32 query rows) per wave in the bf16 prefill tile.
constexpr int kPrefillNCB = 1;

template <typename T, int D>
constexpr int prefill_rows() {
  return sizeof(T) == 2 ? Pf<D, kPrefillNCB>::ROWS : kPrefillRows;
}

template <typename T, int D>
struct MixedSmem {
  static constexpr int PB = sizeof(T) == 2 ? Pf<D, kPrefillNCB>::BYTES : PrefillSmem<T, D>::BYTES;
  static constexpr int BYTES = PB > (int)sizeof(DecodeSmem<T, D>) ? PB : (int)sizeof(DecodeSmem<T, D>);
};

// Mixed launch over the planner's work list.
template <typename T, int D>
__global__ void __launch_bounds__(kThreads, 2) mixed_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[MixedSmem<T, D>::BYTES];
  if ((int)blockIdx.x >= *a.nitems) return;
  const int4 it = a.items[blockIdx.x];
  if (it.x == kItemPrefill) {
    if constexpr (sizeof(T) == 2) {
      prefill_tile_bf16<D, kPrefillNCB>(a, it.y, it.z, it.w, smem);
    } else {
      prefill_tile<T, D>(a, it.y, it.z, it.w, smem);
    }
  } else {
    decode_item<T, D, 1>(a, it.y, it.z, it.w, (long long)a.cu_q[it.y], smem);
  }
}

// Planner: one workgroup of 1024 threads turns (cu_seqlens_q, seq_lens) into
// the work list.  Prefill tiles first (per request and kv head, last tile
// first: the later query rows see more keys), then the chunks of q_len == 1
// requests (per chunk, the kv-head groups); each item is written at its XCD
// dispatch position.
__global__ void __launch_bounds__(1024) plan_kernel(const int32_t* __restrict__ cu_q,
                                                    const int32_t* __restrict__ seq_lens,
                                                    int num_reqs, int hkv, int group, int nhg,
                                                    int kstep, int rows, int len_cap,
                                                    long long max_items,
                                                    int4* __restrict__ items,
                                                    int* __restrict__ count) {
  __shared__ long long s_a[1024];
  __shared__ long long s_b[1024];
  __shared__ long long s_tot[2];
  const int tid = threadIdx.x;
  // pass 1: totals
  long long pf = 0, dc = 0;
  for (int r = tid; r < num_reqs; r += 1024) {
    const int ql = cu_q[r + 1] - cu_q[r];
    if (ql > 1) pf += (long long)hkv * cdiv(ql * group, rows);
    else if (ql == 1) dc += (long long)nhg * num_splits(min(seq_lens[r], len_cap), kstep);
  }
  s_a[tid] = pf;
  s_b[tid] = dc;
  __syncthreads();
  for (int st = 512; st > 0; st >>= 1) {
    if (tid < st) {
      s_a[tid] += s_a[tid + st];
      s_b[tid] += s_b[tid + st];
    }
    __syncthreads();
  }
  const long long total_pf = s_a[0];
  const long long total = s_a[0] + s_b[0];
  __syncthreads();
  // More items than the workspace was sized for means the metadata broke a
  // precondition (total_q or max_seq_len too small): run nothing.
  if (total > max_items) {
    if (tid == 0) *count = 0;
    return;
  }
  if (tid == 0) {
    *count = (int)total;
    s_tot[0] = 0;
    s_tot[1] = 0;
  }
  // pass 2: exclusive scans per chunk of 1024 requests, then emit
  for (int base = 0; base < num_reqs; base += 1024) {
    const int r = base + tid;
    int ql = 0, L = 0;
    long long npf = 0, ndc = 0;
    if (r < num_reqs) {
      ql = cu_q[r + 1] - cu_q[r];
      L = min(seq_lens[r], len_cap);
      if (ql > 1) npf = (long long)hkv * cdiv(ql * group, rows);
      else if (ql == 1) ndc = (long long)nhg * num_splits(L, kstep);
    }
    __syncthreads();
    s_a[tid] = npf;
    s_b[tid] = ndc;
    __syncthreads();
    for (int st = 1; st < 1024; st <<= 1) {  // inclusive Hillis-Steele scan
      const long long xa = tid >= st ? s_a[tid - st] : 0;
      const long long xb = tid >= st ? s_b[tid - st] : 0;
      __syncthreads();
      s_a[tid] += xa;
      s_b[tid] += xb;
      __syncthreads();
    }
    const long long off_pf = s_tot[0] + s_a[tid] - npf;
    const long long off_dc = total_pf + s_tot[1] + s_b[tid] - ndc;
    if (ql > 1) {
      const int tiles = cdiv(ql * group, rows);
      for (int g = 0; g < hkv; ++g)
        for (int k = 0; k < tiles; ++k) {
          const long long l = off_pf + (long long)g * tiles + k;
          items[xcd_position(l, total)] = make_int4(kItemPrefill, r, g, tiles - 1 - k);
        }
    } else if (ql == 1) {
      const int S = num_splits(L, kstep);
      for (int s = 0; s < S; ++s)
        for (int hg = 0; hg < nhg; ++hg) {
          const long long l = off_dc + (long long)s * nhg + hg;
          items[xcd_position(l, total)] = make_int4(kItemDecode, r, hg, s);
        }
    }
    __syncthreads();
    if (tid == 1023) {
      s_tot[0] += s_a[1023];
      s_tot[1] += s_b[1023];
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

static AttnArgs make_args(const AttnHostArgs& h, const WorkspaceLayout& w) {
  AttnArgs a{};
  a.q = h.q;
  a.cu_q = h.cu_seqlens_q;
  a.q_pos = h.q_pos;
  a.k_pool = h.k_pool;
  a.v_pool = h.v_pool;
  a.block_table = h.block_table;
  a.bt_stride = h.block_table_stride;
  a.seq_lens = h.seq_lens;
  a.cu_k = h.cu_seqlens_k;
  a.k_pos = h.k_pos;
  a.cos_tab = h.cos_tab;
  a.sin_tab = h.sin_tab;
  a.max_pos = h.max_pos;
  a.num_reqs = h.num_reqs;
  a.hq = h.hq;
  a.hkv = h.hkv;
  a.group = h.hq / h.hkv;
  a.num_blocks = h.num_blocks;
  a.max_seq_len = h.max_seq_len;
  a.s_max = w.s_max;
  a.nhg = w.nhg;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)h.head_dim));
  a.out = h.out;
  unsigned char* ws = (unsigned char*)h.workspace;
  a.ws_ml = (float2*)(ws + w.ml_off);
  a.ws_o = (float*)(ws + w.o_off);
  a.items = (const int4*)(ws + w.items_off);
  a.nitems = (const int*)(ws + w.count_off);
  return a;
}

template <typename T, int D>
static void launch_combine(const AttnArgs& a, hipStream_t s) {
  if (a.s_max > 1)
    hipLaunchKernelGGL((combine_kernel<T, D>), dim3((unsigned)(a.num_reqs * a.hkv)),
                       dim3(kThreads), 0, s, a);
}

template <typename T, int D>
static int launch_decode(const AttnArgs& a, hipStream_t s) {
  const long long n = (long long)a.num_reqs * a.s_max * a.nhg;
  if (n > 0x7fffffffLL || (long long)a.num_reqs * a.hkv > 0x7fffffffLL) return PIC_EUNSUPPORTED;
  hipLaunchKernelGGL((decode_kernel<T, D>), dim3((unsigned)n), dim3(kThreads), 0, s, a);
  launch_combine<T, D>(a, s);
  return hipGetLastError() == hipSuccess ? PIC_OK : PIC_EHIP;
}

template <typename T, int D>
static int launch_mixed(const AttnArgs& a, const WorkspaceLayout& w, const AttnHostArgs& h,
                        hipStream_t s) {
  if (w.max_items > 0x7fffffffLL) return PIC_EUNSUPPORTED;
  unsigned char* ws = (unsigned char*)h.workspace;
  const int len_cap = (int)min((long long)h.max_seq_len,
                              (long long)h.block_table_stride * kBlockSize);
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, s, h.cu_seqlens_q, h.seq_lens,
                     h.num_reqs, h.hkv, h.hq / h.hkv, w.nhg, Cfg<T, D>::KSTEP,
                     prefill_rows<T, D>(), len_cap,
                     w.max_items, (int4*)(ws + w.items_off), (int*)(ws + w.count_off));
  hipLaunchKernelGGL((mixed_kernel<T, D>), dim3((unsigned)w.max_items), dim3(kThreads), 0, s, a);
  launch_combine<T, D>(a, s);
  return hipGetLastError() == hipSuccess ? PIC_OK : PIC_EHIP;
}

}  // namespace pic

using pic::AttnHostArgs;

extern "C" int pic_attn_decode(const void* q, const int32_t* q_pos, const void* k_pool,
                               const void* v_pool, const int32_t* block_table,
                               int block_table_stride, const int32_t* seq_lens,
                               const int32_t* cu_seqlens_k, const int32_t* k_pos,
                               const float* cos_tab, const float* sin_tab, int max_pos,
                               int num_reqs, int num_q_heads, int num_kv_heads, int head_dim,
                               int block_size, int num_blocks, int max_seq_len, int dtype,
                               void* out, void* workspace, size_t workspace_bytes,
                               void* stream) {
  AttnHostArgs h{q, nullptr, q_pos, k_pool, v_pool, block_table, block_table_stride, seq_lens,
                 cu_seqlens_k, k_pos, cos_tab, sin_tab, max_pos, num_reqs, num_reqs, 1,
                 num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_seq_len,
                 dtype, out, workspace, workspace_bytes};
  int st = pic::check_attn_common(h);
  if (st || num_reqs == 0) return st;
  const pic::WorkspaceLayout w = pic::workspace_layout(num_reqs, num_reqs, max_seq_len,
                                                       num_q_heads, num_kv_heads, head_dim);
  const pic::AttnArgs a = pic::make_args(h, w);
  hipStream_t s = (hipStream_t)stream;
  if (dtype == PIC_BF16)
    return head_dim == 128 ? pic::launch_decode<pic::bf16, 128>(a, s)
                           : pic::launch_decode<pic::bf16, 64>(a, s);
  return head_dim == 128 ? pic::launch_decode<float, 128>(a, s)
                         : pic::launch_decode<float, 64>(a, s);
}

extern "C" int pic_attn_prefill(const void* q, const int32_t* cu_seqlens_q, const int32_t* q_pos,
                                const void* k_pool, const void* v_pool,
                                const int32_t* block_table, int block_table_stride,
                                const int32_t* seq_lens, const int32_t* cu_seqlens_k,
                                const int32_t* k_pos, const float* cos_tab, const float* sin_tab,
                                int max_pos, int num_reqs, int total_q, int max_q_len,
                                int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                                int num_blocks, int max_seq_len, int dtype, void* out,
                                void* workspace, size_t workspace_bytes, void* stream) {
  AttnHostArgs h{q, cu_seqlens_q, q_pos, k_pool, v_pool, block_table, block_table_stride,
                 seq_lens, cu_seqlens_k, k_pos, cos_tab, sin_tab, max_pos, num_reqs, total_q,
                 max_q_len, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                 max_seq_len, dtype, out, workspace, workspace_bytes};
  int st = pic::check_attn_common(h);
  if (st || num_reqs == 0 || total_q == 0) return st;
  if (!cu_seqlens_q || max_q_len < 0) return PIC_EINVAL;
  const pic::WorkspaceLayout w = pic::workspace_layout(num_reqs, total_q, max_seq_len,
                                                       num_q_heads, num_kv_heads, head_dim);
  const pic::AttnArgs a = pic::make_args(h, w);
  hipStream_t s = (hipStream_t)stream;
  if (dtype == PIC_BF16)
    return head_dim == 128 ? pic::launch_mixed<pic::bf16, 128>(a, w, h, s)
                           : pic::launch_mixed<pic::bf16, 64>(a, w, h, s);
  return head_dim == 128 ? pic::launch_mixed<float, 128>(a, w, h, s)
                         : pic::launch_mixed<float, 64>(a, w, h, s);
}
