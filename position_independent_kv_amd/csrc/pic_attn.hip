// Position-free paged attention for gfx950: pic_attn_decode, pic_attn_prefill
// and their rotated-cache variants (key rotation compiled out).
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
//     S^T = K_rot * Q_rot^T      A = rotated keys (keys x d), B = queries
//     O^T += V^T * P^T           A = values transposed (d x keys), B = probs
// Keys are the M dimension of the score tile, so the score accumulator lands
// in exactly the register layout the PV product wants for its B operand (no
// shuffles), and V^T is read straight from the pool because the pool stores
// V transposed inside each block.  The rotation pairs element i with i + d/2;
// in this operand layout both halves of a pair sit in the same lane, so the
// rotation is a handful of FMAs on registers.
//
// Kernels:
// - decode_kernel (batches of q_len == 1, HBM bound): one workgroup of four
//   waves per (request, key chunk of about 512 keys, four kv heads), one wave
//   per kv head, the G query heads of the kv head as the columns of a
//   16x16x32 tile.  The chunk's block ids and positions, and each 32-key
//   step's cos/sin rows (by direct global-to-LDS loads), are staged in LDS
//   once per workgroup; every wave loads its own head's K rows and V runs
//   into registers.  A request split
//   into several chunks writes normalised partials and (max, sum) to the
//   workspace; combine_kernel merges them.
// - plan_kernel + mixed_kernel (any mix of q_len): the planner turns
//   (cu_seqlens_q, seq_lens) into a work list of prefill tiles and decode
//   chunks, and one mixed_kernel launch runs both kinds.  A bf16 prefill tile
//   is one workgroup of eight waves per (request, kv head, 256 query rows:
//   (token, group head) pairs, 32 per wave) on 32x32x16 MFMAs; each 64-key
//   step is gathered from the pool once per workgroup, K rotated on its way
//   into LDS and V^T loaded straight into LDS, and shared by the eight
//   waves.  Its softmax exponentiates against a fixed per-row reference and
//   redoes the tile with the exact row maximum in the rare case a later
//   score overflows that reference.  A
//   launch with few tiles splits long tiles into key chunks, merged by
//   combine_kernel.  fp32 tiles use four waves, 128 rows and an online
//   softmax.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <math.h>

#include <atomic>
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
  int total_q;
  int hq;
  int hkv;
  int group;
  int num_blocks;
  int max_seq_len;
  int s_max;
  int nhg;
  int dec_cpi;       // decode launch: consecutive key chunks per work item (1 or 2)
  float scale_log2;  // log2(e) / sqrt(d): scores are kept in base-2 units
  void* out;
  float2* ws_ml;
  float* ws_o;
  const int4* items;
  const int* nitems;
  // split prefill tiles (null when the launch cannot split): per split item
  // (its work-list position) and row, (max, sum) and the normalised output;
  // the split tiles the merge visits, and their number
  float2* pf_ml;
  float* pf_o;
  int4* pf_tiles;
  int* pf_count;
  // chunk table of the shared-span decode (null elsewhere): chunks per
  // request, and per request s_max + 1 chunk start blocks
  const int* cdc_count;
  const int* cdc_start;
  // decode with append (null elsewhere): row r ([hkv][D]) is request r's new
  // token, its key slot seq_lens[r] - 1
  const void* new_k;
  const void* new_v;
};

// Work item x field: kind in bits 0-3; for a split prefill tile the split
// index in bits 4-15 and the number of splits in bits 16-27 (0: not split).
__host__ __device__ constexpr int item_code(int kind, int split, int nsplit) {
  return kind | (split << 4) | (nsplit << 16);
}
__device__ __forceinline__ int item_kind(int x) { return x & 15; }
__device__ __forceinline__ int item_split(int x) { return (x >> 4) & 0xfff; }
__device__ __forceinline__ int item_nsplit(int x) { return max(1, (x >> 16) & 0xfff); }

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

// Swizzle of a decode table row (D/2 floats in 16-byte units): unit u of key
// row r sits at u ^ tab_swz(r), even, so an 8-float run stays contiguous and
// the rotation's reads (16 key rows per half wave, one column) spread over
// the LDS banks.
__device__ __forceinline__ int tab_swz(int row, int upr) {
  return (2 * ((row & 3) | (((row >> 3) & 1) << 2))) & (upr - 1);
}

// The same rotation with the cos/sin values read from a swizzled LDS table
// row (tab_swz), one chunk at a time: cs/sn point at row `row` of the stage.
template <typename T, int D>
__device__ __forceinline__ void rotate_from_tab(OpT<T>* x, const float* cs, const float* sn,
                                                int row, int grp) {
  using C = Cfg<T, D>;
  using M = Mma<T>;
  typedef Run<float, C::KPL> RF;
  const int f = tab_swz(row, D / 8);
#pragma unroll
  for (int c = 0; c < C::NH; ++c) {
    const int i0 = grp * C::KPL + c * C::KCH;
    const int off = (((i0 >> 2) ^ f) << 2) | (i0 & 3);
    const typename RF::V cv = RF::load(cs + off);
    const typename RF::V sv = RF::load(sn + off);
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
// Largest probability sum of one 32-key block that the prefill tile's first
// pass accepts (2^32): with it no accumulator can overflow for any finite
// bf16 value below 2^70.
constexpr float kPBig = 4294967296.0f;

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
// q heads per kv head whose first-chunk partials a two-chunk decode item can
// hold in LDS until it is done (wider groups take one chunk per item)
constexpr int kStashGroup = 8;

// LDS of a decode workgroup: the chunk's key positions and block ids, and
// the cos/sin rows of two steps (one row per key of the step, padded so the
// 16 rows one read instruction touches fall in different banks).
constexpr int kCdcMaxKeys = kCdcMaxGap * kBlockSize;  // keys of the longest shared-span chunk
static_assert(kCdcMaxKeys <= kMaxChunk, "a shared-span chunk fits the decode's LDS staging");

// chunks of request r (L keys): from the table, or the uniform split
__device__ __forceinline__ int chunks_of(const AttnArgs& a, int r, int L, int kstep) {
  if (a.cdc_count) return min(max(a.cdc_count[r], 1), a.s_max);
  return num_splits(L, kstep);
}

// One 16-byte direct load per lane from global memory into LDS: lane i's
// bytes land at LDS byte address lds_base + 16 i (lds_base: wave-uniform,
// passed in M0, whose previous value the sequence restores).  Inline
// assembly on purpose: the compiler neither counts it nor makes later LDS
// reads wait on it (with the builtin form it may put a wait for every
// outstanding load in front of the step's first LDS read, which serialises
// the load pipeline), so callers wait with vm_wait_all() before the barrier
// that publishes the stage.
__device__ __forceinline__ void lds_direct_load16(const void* src, unsigned lds_base) {
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds_base)
      : "memory");
}
__device__ __forceinline__ void vm_wait_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait until at most N vector-memory loads of this wave are outstanding (loads
// complete in issue order, so every load issued before the last N has landed).
template <int N>
__device__ __forceinline__ void vm_wait_n() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ unsigned lds_address(const void* p) {
  return (unsigned)(size_t)(const __attribute__((address_space(3))) void*)p;
}

template <typename T, int D, int NTAB = 2, int CPI = 1>
struct DecodeSmem {
  static constexpr int NTS = NTAB;        // table stages: steps in flight + 1
  static constexpr int MAXK = CPI * kMaxChunk;  // keys of the longest work item
  static constexpr int KSTEP = Cfg<T, D>::KSTEP;
  static constexpr int TROW = D / 2;      // floats per table row (unpadded: direct-load runs)
  static constexpr int UPR = TROW / 4;    // 16-byte units per row
  static constexpr int RPC = 256 / TROW;  // rows per 1 KiB run
  static constexpr int NCK = KSTEP / RPC; // 1 KiB runs per table and step
  static_assert(KSTEP % RPC == 0, "whole runs per table step");
  float cs[NTS][KSTEP][TROW];
  float sn[NTS][KSTEP][TROW];
  int pos[MAXK];
  int blk[MAXK / kBlockSize + 2];
};

// One decode work item: request r, key chunk s, kv heads hg*NW .. hg*NW+NW-1
// (one per wave of the NW-wave workgroup).  All waves walk the same keys:
// each step's cos/sin rows are fetched once per workgroup, straight into an
// LDS table stage by direct loads (no registers), and shared; every wave
// reads its own head's K rows and V runs from the pools into registers.  NB
// steps of loads are kept in flight (a ring of NB register buffers and
// NB + 1 table stages): the loads of step j+NB are issued as soon as step j
// has consumed its buffer.
// Keeping the table out of registers puts the bf16 kernel of the decode
// launch (two steps in flight) at 230 VGPRs without spills: two workgroups
// share a compute unit.  The
// chunk's block ids and key positions are staged in LDS first, so no
// address lookup ever waits behind the data loads.  With one chunk the wave
// writes the output row; otherwise it writes a normalised partial and
// (max, sum) that combine_kernel merges.  Uniform across the workgroup.
// ROT = false compiles the key rotation out (the pool then holds keys
// already rotated to this request's positions): no positions, no table rows,
// no per-step barrier.  APPEND: the request's new token (a.new_k / a.new_v
// row r) is its key slot L - 1, in the last chunk.  That chunk's workgroup
// stores the token's rows of its heads into the pools (for later calls) and
// keeps them in LDS (s_new: [2][NW][D], K then V), and its last step takes
// key L - 1 from there instead of from the pools, so no workgroup reads
// what another one writes in the same launch.
template <typename T, int D, int NB, int NW, bool ROT, bool APPEND = false, int CPI = 1>
__device__ void decode_item(const AttnArgs& a, int r, int hg, int s, long long qrow,
                            unsigned char* smem_raw, T* s_new = nullptr, int s_cnt = 1,
                            float* s_stash = nullptr) {
  static_assert(CPI == 1 || CPI == 2, "one or two chunks per item");
  using C = Cfg<T, D>;
  using M = Mma<T>;
  typedef typename M::Op Op;
  using SM = DecodeSmem<T, D, NB + 1, CPI>;
  SM& sm = *reinterpret_cast<SM*>(smem_raw);
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int row16 = lane & 15;
  const int grp = lane >> 4;
  constexpr int NTH = NW * 64;
  const int g = hg * NW + wave;
  const bool active = g < a.hkv;
  const int ga = active ? g : 0;  // a valid head for the loads of an idle wave
  const int G = a.group;
  const int L = seq_len_of(a, r);
  const int S = chunks_of(a, r, L, C::KSTEP);
  if (s >= S) return;
  if (L <= 0) {  // empty context: zero output
    if (active) {
      T* out = (T*)a.out + ((size_t)qrow * a.hq + g * G) * D;
      for (int e = lane; e < G * D; e += 64) out[e] = (T)0.0f;
    }
    return;
  }
  // chunks s .. s_last, walked as one key range; each chunk's (m, l, o) is
  // written as its own partial, so the result is the same as with one chunk
  // per item
  const int s_last = CPI > 1 ? min(s + s_cnt, S) - 1 : s;
  int k0, k1;
  if (a.cdc_start) {  // block-aligned chunk from the table, at most kCdcMaxKeys keys
    const int* st = a.cdc_start + (size_t)r * (a.s_max + 1);
    const int nb = cdiv(L, kBlockSize);
    k0 = min(max(st[s], 0), nb) * kBlockSize;
    k1 = min(min(L, min(max(st[s + 1], 0), nb) * kBlockSize), k0 + kCdcMaxKeys);
    if (k1 <= k0) return;
  } else {
    k0 = chunk_start(L, s, C::KSTEP);
    k1 = chunk_start(L, s_last + 1, C::KSTEP);
  }
  const int nsteps = cdiv(k1 - k0, C::KSTEP);
  // first step of chunk s + 1 (chunk starts are whole steps)
  const int jsplit = s_last > s ? (chunk_start(L, s + 1, C::KSTEP) - k0) / C::KSTEP : nsteps;

  // append: the new token's K and V elements this thread stores (below)
  const bool append = APPEND && s_last == S - 1;
  constexpr int kNewPerThread = APPEND ? (NW * D + NTH - 1) / NTH : 1;
  T new_kx[kNewPerThread], new_vx[kNewPerThread];
  if (append) {
    const T* nk = (const T*)a.new_k + (size_t)r * a.hkv * D;
    const T* nv = (const T*)a.new_v + (size_t)r * a.hkv * D;
#pragma unroll
    for (int i = 0; i < kNewPerThread; ++i) {
      const int e = tid + i * NTH;
      const int gw = hg * NW + e / D;
      if (e < NW * D && gw < a.hkv) {
        new_kx[i] = nk[(size_t)gw * D + e % D];
        new_vx[i] = nv[(size_t)gw * D + e % D];
      }
    }
  }

  // chunk metadata -> LDS: positions of keys k0.., block ids of blocks k0/16..
  {
    const int32_t* bt = a.block_table + (size_t)r * a.bt_stride;
    const int nk = nsteps * C::KSTEP;
    if constexpr (ROT) {
      const int32_t* kp = a.k_pos + a.cu_k[r];
      for (int j = tid; j < nk; j += NTH)
        sm.pos[j] = clampi(kp[min(k0 + j, L - 1)], 0, a.max_pos - 1);
    }
    const int nbk = nk / kBlockSize;
    for (int j = tid; j < nbk; j += NTH)
      sm.blk[j] = clampi(bt[min((k0 >> 4) + j, (L - 1) >> 4)], 0, a.num_blocks - 1);
  }

  Op qop[C::NC];
  const bool qvalid = row16 < G;
  load_query<T, D>(a, qrow, ga * G + (qvalid ? row16 : 0), a.q_pos[qrow], qvalid, grp, qop);
  // append: the new token's rows of this workgroup's heads into LDS (their
  // loads were issued before the chunk's metadata, so their latency overlaps
  // it); they go to the pools once the item is done
  if (append) {
#pragma unroll
    for (int i = 0; i < kNewPerThread; ++i) {
      const int e = tid + i * NTH;
      if (e < NW * D && hg * NW + e / D < a.hkv) {
        s_new[e] = new_kx[i];
        s_new[NW * D + e] = new_vx[i];
      }
    }
  }
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


  struct Group {
    Op k[C::NT][C::NC];
    Op v[C::NPV][C::ND];
  };
  Group grpbuf[NB];

  // Loads of step j (relative to k0) into a register group, in two parts so
  // that each is issued as soon as the previous step has consumed that part
  // of the group: the K rows after the score MFMAs, the V runs after the PV
  // MFMAs.
  // The cos/sin rows of step j straight into table stage j % (NB + 1) (no
  // registers): wave w fills 1 KiB runs w, w + NW, ... of each table.  Issued
  // before that step's K loads: a wave's loads complete in order, so once its
  // K registers are in, so are its table runs.  The stage was last read in
  // step j - NB - 1, which every wave has left: the stage is refilled during
  // step j - NB, after that step's barrier.
  auto dma_tab = [&](int j) {
    const int buf = j % SM::NTS;
    const unsigned cbase = __builtin_amdgcn_readfirstlane(lds_address(&sm.cs[buf][0][0]));
    const unsigned sbase = __builtin_amdgcn_readfirstlane(lds_address(&sm.sn[buf][0][0]));
    const int w = __builtin_amdgcn_readfirstlane(wave);  // uniform: runs per wave
    for (int ck = w; ck < SM::NCK; ck += NW) {
      const int row = ck * SM::RPC + lane / SM::UPR;
      const int unit = (lane % SM::UPR) ^ tab_swz(row, SM::UPR);
      const size_t at = (size_t)sm.pos[j * C::KSTEP + row] * (D / 2) + unit * 4;
      lds_direct_load16(a.cos_tab + at, cbase + ck * 1024u);
      lds_direct_load16(a.sin_tab + at, sbase + ck * 1024u);
    }
  };
  // wait until this wave's K registers of the current step are in (and with
  // them its earlier table runs)
  auto wait_k = [&](Group& gb) {
#pragma unroll
    for (int t = 0; t < C::NT; ++t)
#pragma unroll
      for (int c = 0; c < C::NC; ++c) asm volatile("" ::"v"(gb.k[t][c]));
  };
  auto issue_k = [&](int j, Group& gb) {
    const int kb = j * C::KSTEP;  // offset in the chunk
    const int blk = sm.blk[min((kb >> 4) + kblk_sel, nsteps * C::KSTEP / kBlockSize - 1)];
#pragma unroll
    for (int t = 0; t < C::NT; ++t) {
      const int kk = key_of<C::NT>(t, row16);
      const T* krow = kpool + (size_t)blk * blk_stride + head_k +
                      (size_t)((kb + kk) & 15) * D + grp * C::KPL;
#pragma unroll
      for (int c = 0; c < C::NC; ++c) gb.k[t][c] = M::load(krow + c * C::KCH);
    }
  };
  auto issue_v = [&](int j, Group& gb) {
    const int kb = j * C::KSTEP;
    const int blk = sm.blk[min((kb >> 4) + vblk_sel, nsteps * C::KSTEP / kBlockSize - 1)];
#pragma unroll
    for (int mi = 0; mi < C::NPV; ++mi) {
      const T* vrow = vpool + (size_t)blk * blk_stride + head_v + (size_t)row16 * kBlockSize +
                      ((vkey_off + mi * C::KPL) & 15);
#pragma unroll
      for (int dt = 0; dt < C::ND; ++dt) gb.v[mi][dt] = M::load(vrow + (size_t)dt * 16 * kBlockSize);
    }
  };
  auto issue = [&](int j, Group& gb) {
    if constexpr (ROT) dma_tab(j);
    issue_k(j, gb);
    issue_v(j, gb);
  };

  f32x4 acc[C::ND];
#pragma unroll
  for (int dt = 0; dt < C::ND; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;

  // chunk sc done: its normalised output (a single-chunk request) or its
  // partial (o / l, and (m, l)) for the merge; to_stash: the partial goes to
  // this wave's LDS stash instead and is stored once the item is done (global
  // stores in the middle of the load pipeline measured ~3% on a decode step)
  auto finish = [&](int sc, bool to_stash) {
    const float l_tot = col_sum(l_run);
    if (!active || row16 >= G) return;
    const float inv = 1.0f / l_tot;
    if (to_stash) {
      float* st = s_stash + ((size_t)wave * kStashGroup + row16) * (D + 2);
#pragma unroll
      for (int dt = 0; dt < C::ND; ++dt)
        *reinterpret_cast<f32x4*>(st + dt * 16 + grp * 4) = acc[dt] * inv;
      if (grp == 0) {
        st[D] = m_run;
        st[D + 1] = l_tot;
      }
      return;
    }
    if (S == 1) {
      T* out = (T*)a.out + ((size_t)qrow * a.hq + g * G + row16) * D + grp * 4;
#pragma unroll
      for (int dt = 0; dt < C::ND; ++dt) store4<T>(out + dt * 16, acc[dt], inv);
      return;
    }
    const size_t pidx = (((size_t)r * a.hkv + g) * a.s_max + sc) * G + row16;
    float* po = a.ws_o + pidx * D + grp * 4;
#pragma unroll
    for (int dt = 0; dt < C::ND; ++dt) *reinterpret_cast<f32x4*>(po + dt * 16) = acc[dt] * inv;
    if (grp == 0) a.ws_ml[pidx] = make_float2(m_run, l_tot);
  };

#pragma unroll
  for (int b = 0; b < NB; ++b)
    if (b < nsteps) issue(b, grpbuf[b]);

  // step j with its loads in group gb; buf: LDS table stage
  auto step = [&](int j, Group& gb) {
    const int buf = j % SM::NTS;
    const int kb = k0 + j * C::KSTEP;  // absolute key index
    if constexpr (CPI > 1) {
      if (j == jsplit) {  // chunk s ends: its partial, then a fresh state for chunk s + 1
        finish(s, s_stash != nullptr && G <= kStashGroup);
#pragma unroll
        for (int dt = 0; dt < C::ND; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        m_run = -INFINITY;
        l_run = 0.0f;
      }
    }
    if constexpr (ROT) {
      wait_k(gb);
      __syncthreads();
    }
    if (append && j == nsteps - 1) {  // key L - 1: the new token's K, before its rotation
#pragma unroll
      for (int t = 0; t < C::NT; ++t)
        if (kb + key_of<C::NT>(t, row16) == L - 1)
#pragma unroll
          for (int c = 0; c < C::NC; ++c)
            gb.k[t][c] = M::load(s_new + wave * D + grp * C::KPL + c * C::KCH);
    }
    f32x4 sc[C::NT];
#pragma unroll
    for (int t = 0; t < C::NT; ++t) {
      const int krow = key_of<C::NT>(t, row16);
      if constexpr (ROT)
        rotate_from_tab<T, D>(gb.k[t], &sm.cs[buf][krow][0], &sm.sn[buf][krow][0], krow, grp);
      sc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < C::NC; ++c) sc[t] = M::run(gb.k[t][c], qop[c], sc[t]);
    }
    if (j + NB < nsteps) {
      if constexpr (ROT) dma_tab(j + NB);
      issue_k(j + NB, gb);
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
      if (append && nvalid >= 1 && nvalid <= C::KPL) {  // this run holds key L - 1
#pragma unroll
        for (int dt = 0; dt < C::ND; ++dt)
          M::set(gb.v[mi][dt], nvalid - 1, (float)s_new[(NW + wave) * D + row16 + 16 * dt]);
      }
    }
#pragma unroll
    for (int mi = 0; mi < C::NPV; ++mi) {
      const Op p = pack_probs<T, D>(sc, mi);
#pragma unroll
      for (int dt = 0; dt < C::ND; ++dt) acc[dt] = M::run(gb.v[mi][dt], p, acc[dt]);
    }
    if (j + NB < nsteps) issue_v(j + NB, gb);
  };

  for (int j0 = 0; j0 < nsteps; j0 += NB) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
      if (j0 + b < nsteps) step(j0 + b, grpbuf[b]);
  }

  // append: the new token into the pools, for later calls (nothing in this
  // launch reads it there; a block id out of range is not written)
  if (append) {
    const int blk = a.block_table[(size_t)r * a.bt_stride + ((L - 1) >> 4)];
    const int off = (L - 1) & 15;
    if (blk >= 0 && blk < a.num_blocks) {
      T* kpw = (T*)a.k_pool;
      T* vpw = (T*)a.v_pool;
      for (int e = tid; e < NW * D; e += NTH) {
        const int gw = hg * NW + e / D, d = e % D;
        if (gw < a.hkv) {
          kpw[(((size_t)blk * a.hkv + gw) * kBlockSize + off) * D + d] = s_new[e];
          vpw[(((size_t)blk * a.hkv + gw) * D + d) * kBlockSize + off] = s_new[NW * D + e];
        }
      }
    }
  }
  finish(s_last, false);
  if (CPI > 1 && s_stash && G <= kStashGroup && jsplit < nsteps && active &&
      row16 < G) {  // chunk s's partial, from the stash
    const float* st = s_stash + ((size_t)wave * kStashGroup + row16) * (D + 2);
    const size_t pidx = (((size_t)r * a.hkv + g) * a.s_max + s) * G + row16;
    float* po = a.ws_o + pidx * D + grp * 4;
#pragma unroll
    for (int dt = 0; dt < C::ND; ++dt)
      *reinterpret_cast<f32x4*>(po + dt * 16) = *reinterpret_cast<const f32x4*>(st + dt * 16 + grp * 4);
    if (grp == 0) a.ws_ml[pidx] = make_float2(st[D], st[D + 1]);
  }
}

// Merge the chunk partials of every multi-chunk q_len == 1 request:
// o = sum_s w_s o_s / sum_s w_s with w_s = l_s 2^(m_s - max m).  One
// workgroup per (request, kv head); threads take (column, 8 consecutive d)
// pairs, and threads beyond those pairs take every SG-th chunk in parallel.
// Merge of one quarter of d of one split prefill tile (kPrefillTileRows
// threads, one query row each): o = sum_s w_s o_s / sum_s w_s with
// w_s = l_s 2^(m_s - max m), over the tile's chunks that saw a key of the
// row (every row sees key 0, so at least the first chunk).  All chunks'
// (m, l) are read first, then the partial rows, so no load waits on another
// (a running rescale chained every chunk's loads behind the previous
// chunk's, and the merge of a few long-context tiles took 20-30 us).  A
// chunk that saw no key of the row may hold stale values: a select skips
// it, nothing multiplies them.
constexpr int kMergeParts = 4;
template <typename T, int D>
__device__ void merge_prefill_tile(const AttnArgs& a, int idx, int part) {
  static_assert(kThreads == kPrefillTileRows, "one thread per tile row");
  static_assert(D % (4 * kMergeParts) == 0, "whole f32x4 pieces per part");
  constexpr int NQ = D / kMergeParts / 4;  // f32x4 pieces of this part
  if (!a.pf_tiles || idx >= *a.pf_count) return;
  const int4 t = a.pf_tiles[idx];  // request, kv head, tile, first item
  const int r = t.x, g = t.y, p0 = t.w;
  if (r < 0 || r >= a.num_reqs || g < 0 || g >= a.hkv || p0 < 0 || p0 >= kSplitCUs) return;
  const int S = min(item_nsplit(a.items[p0].x), kSplitCUs - p0);
  const int q0 = a.cu_q[r];
  const int ql = a.cu_q[r + 1] - q0;
  const int G = a.group;
  const int n = t.z * kPrefillTileRows + (int)threadIdx.x;
  if (n >= ql * G) return;
  const size_t row0 = (size_t)p0 * kPrefillTileRows + threadIdx.x;
  float m = -INFINITY;
#pragma unroll 4
  for (int s = 0; s < S; ++s) {
    const float2 ml = a.pf_ml[row0 + (size_t)s * kPrefillTileRows];
    if (ml.y > 0.0f) m = fmaxf(m, ml.x);
  }
  float l = 0.0f;
  f32x4 o[NQ];
#pragma unroll
  for (int e = 0; e < NQ; ++e) o[e] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int s = 0; s < S; ++s) {
    const size_t prow = row0 + (size_t)s * kPrefillTileRows;
    const float2 ml = a.pf_ml[prow];
    const f32x4* src = reinterpret_cast<const f32x4*>(a.pf_o + prow * D) + part * NQ;
    f32x4 x[NQ];
#pragma unroll
    for (int e = 0; e < NQ; ++e) x[e] = src[e];
    const bool seen = ml.y > 0.0f;
    const float w = seen ? ml.y * fast_exp2(ml.x - m) : 0.0f;
    l += w;
#pragma unroll
    for (int e = 0; e < NQ; ++e) o[e] = seen ? o[e] + x[e] * w : o[e];
  }
  const float inv = 1.0f / l;
  T* dst = (T*)a.out + (((size_t)q0 + n / G) * a.hq + g * G + n % G) * D + part * NQ * 4;
#pragma unroll
  for (int e = 0; e < NQ; ++e) store4<T>(dst + 4 * e, o[e], inv);
}

// NaN into the output rows of request r for the q heads of kv head g (rows
// clipped to [0, total_q)): what a mixed launch leaves when its planner
// refused a work list larger than the workspace.
template <typename T, int D>
__device__ void fill_nan_rows(const AttnArgs& a, int r, int g) {
  const int q0 = max(a.cu_q[r], 0), q1 = min(a.cu_q[r + 1], a.total_q);
  const int G = a.group;
  const long long n = (long long)max(q1 - q0, 0) * G * D;
  T* out = (T*)a.out;
  for (long long i = threadIdx.x; i < n; i += kThreads) {
    const long long row = q0 + i / (G * D);
    const int h = g * G + (int)((i / D) % G);
    out[(row * a.hq + h) * D + i % D] = (T)__builtin_nanf("");
  }
}

// Blocks [0, dec_blocks): dsplit per (request, kv head), each merging the
// chunks of a q_len == 1 request for one slice of d (or, after a refused
// work list, the first filling the request's rows with NaN); blocks beyond:
// kMergeParts per split prefill tile, one per quarter of d.
template <typename T, int D>
__global__ void __launch_bounds__(kThreads) combine_kernel(AttnArgs a, int dec_blocks,
                                                           int dsplit) {
  constexpr int EPT = 8;
  __shared__ __attribute__((aligned(16))) float gm[kThreads * EPT];
  __shared__ float2 gml[kThreads];
  const int tid = threadIdx.x;
  if ((int)blockIdx.x >= dec_blocks) {
    if constexpr (sizeof(T) == 2) {
      const int b = (int)blockIdx.x - dec_blocks;
      merge_prefill_tile<T, D>(a, b / kMergeParts, b % kMergeParts);
    }
    return;
  }
  const int rg = (int)blockIdx.x / dsplit, ds = (int)blockIdx.x % dsplit;
  const int r = rg / a.hkv;
  const int g = rg % a.hkv;
  if (a.cu_q && a.nitems[1]) {  // the planner ran nothing (work list overflow)
    if (ds == 0) fill_nan_rows<T, D>(a, r, g);
    return;
  }
  if (a.cu_q && a.cu_q[r + 1] - a.cu_q[r] != 1) return;
  const long long qrow = a.cu_q ? (long long)a.cu_q[r] : (long long)r;
  const int L = seq_len_of(a, r);
  const int S = chunks_of(a, r, L, Cfg<T, D>::KSTEP);
  if (L <= 0 || S <= 1) return;
  const int G = a.group;
  const int DE = D / EPT / dsplit;  // EPT-wide d pieces of this block's slice
  const int pairs = G * DE;
  const int SG = max(1, kThreads / pairs);
  const int sg = tid / pairs;
  const int pc = tid % pairs;
  const int col = pc / DE;
  const int d0 = (ds * DE + pc % DE) * EPT;
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
// [tile*ROWS, tile*ROWS + ROWS), ROWS = 32 per wave
// ---------------------------------------------------------------------------

// Swizzle of the V^T stage: row r's unit u sits at slot u ^ vswz(r), so the
// PV operand reads (32 rows, one unit each, per half wave) and the direct
// loads (8 rows x 8 units per 64 lanes) hit distinct LDS banks.
__device__ __forceinline__ int vswz(int r) { return (r ^ ((r >> 3) & 3)) & 7; }

template <int D, int NW, int KS>
struct Pf {
  static constexpr int NTH = NW * 64;              // threads
  static constexpr int KSTEP = KS;                 // keys per step
  static constexpr int NBLK = KS / 32;             // 32-key blocks per step
  static constexpr int ROWS = NW * 32;             // query rows per tile
  static constexpr int NCH = D / 16;               // 16-wide d chunks (MFMA K)
  static constexpr int NHC = NCH / 2;              // chunks of the first half of d
  static constexpr int NDB = D / 32;               // 32-row d blocks of O^T
  static constexpr int KLD = D + 8;                // LDS K row stride (bf16)
  static constexpr int VLD = KSTEP;                // LDS V^T row length (bf16), swizzled
  static constexpr int QLD = D + 8;                // LDS row stride of the query operand
  static constexpr int KBUF = KSTEP * KLD;         // bf16 elements of one K stage
  static constexpr int VBUF = D * VLD;             // bf16 elements of one V^T stage
  static constexpr int NKB = 3, NVB = 2;           // K and V^T stages
  static constexpr int V_OFF = NKB * KBUF;
  static constexpr int Q_OFF = V_OFF + NVB * VBUF;
  static constexpr int BYTES = (Q_OFF + ROWS * QLD) * 2;
  static constexpr int KPT = KSTEP * (D / 2) / NTH;  // rotation pairs per thread
  static constexpr int KTPK = (D / 2) / KPT;         // threads per key
  // V^T stage: D rows x 64 keys as 16-byte units (8 keys), unit u of row
  // r at position 8r + (u ^ vswz(r)); each wave fills NDMA runs of 64 units
  static constexpr int NDMA = D * KSTEP * 2 / (NW * 64 * 16);
  static_assert(KPT % 4 == 0 && KPT <= D / 2, "whole 8-byte K pieces per thread");
};

// One prefill tile, bf16, software-pipelined over 32-key blocks: the score
// MFMAs of block b+1 do not depend on the exponentials of block b or on its
// PV MFMAs, so matrix and vector work can overlap, within a wave and between
// the two waves of a SIMD (the instruction order is the compiler's).
//
// Staging: each 64-key step is gathered from the paged pools once per
// workgroup.  Every thread loads its share of K rows and cos/sin rows into
// registers right after it has rotated the previous ones into LDS, a whole
// step before they are rotated in turn (in the step's second half); K is
// rotated on the way into LDS.  V^T needs no arithmetic, so it goes from the
// pool straight into LDS (16-byte direct loads, no registers, no LDS write
// instructions).  K is
// staged two steps ahead (three K stages: the block being exponentiated may
// be re-read, the next block is being multiplied, and the step after is
// being written), V^T one step ahead (two stages).
// One barrier per step.  The rotated query rows (the B operand, pre-scaled
// by log2(e)/sqrt(d) so scores come out in base-2 units) sit in a per-wave
// LDS slice.  Steps that lie wholly below the causal diagonal skip the mask.
template <int D, int NW, int KS, bool ROT>
__device__ void prefill_tile_bf16(const AttnArgs& a, int r, int g, int tile, int split,
                                  int nsplit, int pslot, unsigned char* smem) {
  using P = Pf<D, NW, KS>;
  static_assert(P::KSTEP == 64 && P::NDMA >= 1 && P::NDMA <= 2 &&
                    P::NDMA * NW * 64 * 8 == D * P::KSTEP,
                "V^T stages fill in whole 1 KiB direct-load runs per wave");
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
  // keys [kofs, kstop) of this item: the whole range, or chunk `split` of
  // nsplit equal chunks of whole steps
  int kofs = 0, kstop = kend;
  if (nsplit > 1) {
    const int chunk = cdiv(cdiv(kend, nsplit), P::KSTEP) * P::KSTEP;
    kofs = min(kend, split * chunk);
    kstop = min(kend, kofs + chunk);
  }
  const int nsteps = cdiv(kstop - kofs, P::KSTEP);
  bf16* const lds = reinterpret_cast<bf16*>(smem);

  // query row of this lane's column, its causal limit, and its LDS slice
  const int n = trow0 + wave * 32 + col;
  const bool valid = n < nrows;
  const int tok = (valid ? n : 0) / G;
  const int head = (valid ? n : 0) % G;
  const int lim = valid ? L - ql + tok : -1;  // last visible key slot of this row
  bf16* const qs = lds + P::Q_OFF + (wave * 32 + col) * P::QLD + hh * 8;
  // The query row and its position are loaded here; the table rows and the
  // rotation into LDS come in the first prologue, so that the row's loads,
  // the first steps' block lookups and then their K/V loads are all in
  // flight together (a tile's start otherwise waits on a chain of dependent
  // loads, and a workgroup fills its compute unit alone).
  Op qop[P::NCH];
  {
    const bf16* qp = (const bf16*)a.q + (((size_t)q0 + tok) * a.hq + g * G + head) * D + hh * 8;
#pragma unroll
    for (int c = 0; c < P::NCH; ++c) qop[c] = *reinterpret_cast<const Op*>(qp + c * 16);
  }
  const int qpos = clampi(a.q_pos[q0 + tok], 0, a.max_pos - 1);

  const int32_t* bt = a.block_table + (size_t)r * a.bt_stride;
  const int32_t* kp = ROT ? a.k_pos + a.cu_k[r] : nullptr;
  const int nb_max = a.num_blocks - 1;
  const int pmax = a.max_pos - 1;
  const size_t blk_bytes = (size_t)a.hkv * kBlockSize * D * sizeof(bf16);

  // staging: thread -> (key skey, pairs si0..si0+KPT) for K and the table,
  // V^T units as below.  Every step starts at a multiple of 64, so a thread
  // always reads the same row of a block (skey % 16) and the same units of
  // V^T: the per-step address is block base plus a fixed per-thread offset.
  // A key at or beyond L reads a valid slot of the last block (its score is
  // masked, its V zeroed); a step past the end re-reads valid slots and is
  // never used.
  const int skey = tid / P::KTPK;
  const int si0 = (tid % P::KTPK) * P::KPT;
  // V^T direct loads: the wave fills LDS runs vrun0 .. vrun0 + NDMA - 1 (64
  // units each, in slot order); in run i this lane's unit is row
  // vrow0 + 8i, unit vu ^ i (the swizzle of row vrow0 + 8i is that of vrow0
  // with bit 0 flipped), so both of its units lie in the same 16-key block
  const int vrun0 = P::NDMA * wave;
  const int vrow0 = vrun0 * 8 + (lane >> 3);
  const int vu = (lane & 7) ^ vswz(vrow0);
  const int vbi = vu >> 1;  // block of the step this lane's units lie in
  const char* kthr = (const char*)a.k_pool +
                     (((size_t)g * kBlockSize + (skey & 15)) * D + si0) * sizeof(bf16);
  const char* cthr = (const char*)(a.cos_tab + si0);
  const char* sthr = (const char*)(a.sin_tab + si0);
  const char* vthr = (const char*)a.v_pool + ((size_t)g * D + vrow0) * kBlockSize * sizeof(bf16);
  const unsigned v_lds0 = __builtin_amdgcn_readfirstlane(
      lds_address(lds + P::V_OFF) + (unsigned)vrun0 * 1024u);
  typedef vec<bf16, P::KPT> KV;
  typedef vec<float, P::KPT> TV;
  struct KRegs {
    KV lo, hi;  // unrotated halves of the thread's K piece
    TV c, s;    // their cos/sin
  };
  KRegs kr;
  // vector-memory loads issued by one kmeta() and by one kload(), at least:
  // a load instruction moves at most 16 bytes, so the compiler can only
  // issue more, and a counted wait below (at most N loads outstanding, in
  // issue order) then waits for more than it needs, never for less.  The
  // direct-load and wait statements are compiler barriers for memory
  // accesses, so these loads stay between them.
  constexpr int kMetaLoads = ROT ? 2 : 1;
  constexpr int kDataLoads = 2 + (ROT ? 2 * cdiv(P::KPT * 4, 16) : 0);
  // Addresses (block ids, position) of the next loads, looked up before
  // those loads are issued: kmeta_* / vmeta_* hold the ones in use, the *_nx
  // copies the ones being fetched.  Lookups are issued at the top of a step,
  // before its V direct loads, and used at the end of the step (K) or at
  // the top of the next (V).
  int kmeta_blk, kmeta_pos, vmeta_blk;
  int kmeta_blk_nx, kmeta_pos_nx = 0, vmeta_blk_nx;
  auto kmeta = [&](int kb) {  // kb: absolute key index of a step's first key
    const int kc = min(kb + skey, L - 1);
    kmeta_blk_nx = bt[kc >> 4];
    if constexpr (ROT) kmeta_pos_nx = kp[kc];
  };
  auto vmeta = [&](int kb) {
    vmeta_blk_nx = bt[min(kb + 16 * vbi, L - 1) >> 4];
  };
  auto kmeta_use = [&]() {
    kmeta_blk = kmeta_blk_nx;
    kmeta_pos = kmeta_pos_nx;
  };
  auto vmeta_use = [&]() {
    vmeta_blk = vmeta_blk_nx;
  };
  // the (block, position) of key kb + skey, looked up without touching the
  // pipeline's *_nx registers
  auto kmeta_now = [&](int kb, int& blk, int& pos) {
    const int kc = min(kb + skey, L - 1);
    blk = bt[kc >> 4];
    pos = ROT ? kp[kc] : 0;
  };
  auto kload_to = [&](KRegs& d, int kblk, int kpos) {
    // an out-of-range id (negative ones wrap to large unsigned values) is
    // clamped to the last valid one
    const unsigned blk = min((unsigned)kblk, (unsigned)nb_max);
    const unsigned pos = min((unsigned)kpos, (unsigned)pmax);
    const char* src = kthr + (size_t)blk * blk_bytes;
    d.lo = *reinterpret_cast<const KV*>(src);
    d.hi = *reinterpret_cast<const KV*>(src + D);  // + D/2 elements
    if constexpr (ROT) {
      d.c = *reinterpret_cast<const TV*>(cthr + (size_t)pos * (D * 2));  // D/2 floats per row
      d.s = *reinterpret_cast<const TV*>(sthr + (size_t)pos * (D * 2));
    }
  };
  auto kload = [&]() { kload_to(kr, kmeta_blk, kmeta_pos); };
  // V^T of step `step` straight into its LDS stage (no registers)
  auto vdma = [&](int step) {
    const unsigned vb = min((unsigned)vmeta_blk, (unsigned)nb_max);
    const char* src = vthr + (size_t)vb * blk_bytes;
    const unsigned dst = v_lds0 + (unsigned)((step % P::NVB) * P::VBUF * 2);
#pragma unroll
    for (int i = 0; i < P::NDMA; ++i)  // run i: 8 rows further, unit vu ^ i
      lds_direct_load16(src + (i * 8 * kBlockSize + 8 * ((vu ^ i) & 1)) * sizeof(bf16),
                        dst + i * 1024u);
  };
  auto kstore_from = [&](int step, const KRegs& d) {  // rotate a K piece into K stage `step`
    KV lo = d.lo, hi = d.hi;
    if constexpr (ROT) {
#pragma unroll
      for (int e = 0; e < P::KPT; ++e) {
        const float x = (float)d.lo[e], y = (float)d.hi[e];
        lo[e] = (bf16)(x * d.c[e] - y * d.s[e]);
        hi[e] = (bf16)(y * d.c[e] + x * d.s[e]);
      }
    }
    bf16* kd = lds + (step % P::NKB) * P::KBUF + skey * P::KLD + si0;
    *reinterpret_cast<KV*>(kd) = lo;
    *reinterpret_cast<KV*>(kd + D / 2) = hi;
  };
  auto kstore = [&](int step) { kstore_from(step, kr); };
  // Slots at or beyond L hold no data: once this lane's own direct loads
  // into V stage `step` have landed (the caller waits for them), it
  // overwrites those keys of its units with zeros (only the last step has
  // any).
  auto vfix = [&](int step) {
    const int kb = kofs + step * P::KSTEP;
    if (kb + P::KSTEP > L) {
      bf16* vdst = lds + P::V_OFF + (step % P::NVB) * P::VBUF + (vrun0 * 64 + lane) * 8;
#pragma unroll
      for (int i = 0; i < P::NDMA; ++i) {
        const int key0 = kb + 8 * (vu ^ i);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (key0 + e >= L) vdst[i * 512 + e] = (bf16)0.0f;
      }
    }
  };

  // S^T - m of one 32-key block (h) of K stage `step` (negm: -m in every
  // element, the chain's start), d chunk by d chunk, the operands of chunk
  // c+1 read while chunk c multiplies
  auto qk_block = [&](int step, int h, const Acc& negm) {
    const bf16* kr = lds + (step % P::NKB) * P::KBUF + (h * 32 + key32(col)) * P::KLD + hh * 8;
    Op ka = *reinterpret_cast<const Op*>(kr);
    Op qb = *reinterpret_cast<const Op*>(qs);
    Acc sc = negm;
#pragma unroll
    for (int c = 0; c < P::NCH; ++c) {
      Op nka, nqb;
      if (c + 1 < P::NCH) {
        nka = *reinterpret_cast<const Op*>(kr + (c + 1) * 16);
        nqb = *reinterpret_cast<const Op*>(qs + (c + 1) * 16);
      }
      sc = Mma32::run(ka, qb, sc);
      if (c + 1 < P::NCH) {
        ka = nka;
        qb = nqb;
      }
    }
    return sc;
  };
  // C element v of this lane holds key kb + 8*hh + kc(v) of the block (kc: a
  // compile-time constant, from key32)
  auto mask_block = [&](Acc& sc, int kb) {  // kb: first key of the block
    const int t = lim - kb - 8 * hh;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int kc = 16 * (v >> 3) + 4 * ((v >> 2) & 1) + (v & 3);
      if (kc > t) sc[v] = -INFINITY;
    }
  };
  auto col_max = [&](const Acc& sc) {
    float mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sc[v]);
    return fmaxf(mx, __shfl_xor(mx, 32));
  };
  // The first K stages and V stage (and, with_q, the rotated queries), and
  // the next loads' addresses.  Every lookup is issued first, then every
  // data load, then the stores: two memory round trips, not a chain of six.
  auto prologue = [&](bool with_v, bool with_q) {
    int b0, p0, b1, p1;
    kmeta_now(kofs, b0, p0);
    kmeta_now(kofs + P::KSTEP, b1, p1);
    if (with_v) vmeta(kofs);
    vec<float, 8> qc[P::NHC], qsn[P::NHC];
    if (with_q) {
      const float* cr = a.cos_tab + (size_t)qpos * (D / 2) + hh * 8;
      const float* sr = a.sin_tab + (size_t)qpos * (D / 2) + hh * 8;
#pragma unroll
      for (int c = 0; c < P::NHC; ++c) {
        qc[c] = *reinterpret_cast<const vec<float, 8>*>(cr + c * 16);
        qsn[c] = *reinterpret_cast<const vec<float, 8>*>(sr + c * 16);
      }
    }
    KRegs k1;
    kload_to(kr, b0, p0);
    kload_to(k1, b1, p1);
    if (with_v) {
      vmeta_use();
      vdma(0);
    }
    kmeta(kofs + 2 * P::KSTEP);
    if (with_v) vmeta(kofs + P::KSTEP);
    if (with_q) {
#pragma unroll
      for (int c = 0; c < P::NHC; ++c) {
        float lo[8], hi[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = (float)qop[c][e], y = (float)qop[c + P::NHC][e];
          lo[e] = (x * qc[c][e] - y * qsn[c][e]) * a.scale_log2;
          hi[e] = (y * qc[c][e] + x * qsn[c][e]) * a.scale_log2;
        }
        *reinterpret_cast<Op*>(qs + c * 16) = valid ? Mma<bf16>::pack(lo) : Mma<bf16>::zero();
        *reinterpret_cast<Op*>(qs + (c + P::NHC) * 16) =
            valid ? Mma<bf16>::pack(hi) : Mma<bf16>::zero();
      }
    }
    kstore_from(0, kr);
    kstore_from(1, k1);
    // K step 2 is loaded here and rotated in the first step (each step
    // rotates the K data loaded at the end of the step before)
    kmeta_use();
    kload();
    if (with_v) {
      // V step 0 has landed: after its direct loads came one K lookup, one
      // V lookup and one K step's data
      vm_wait_n<kMetaLoads + 1 + kDataLoads>();
      vfix(0);
    }
    __syncthreads();
  };
  // steps below every row's diagonal (kofs is a multiple of the step)
  const int jfull = min(nsteps, max(0, kfull - kofs) / P::KSTEP);

  // Exact column max over all visible keys (only for the rare second pass).
  auto row_max = [&]() {
    float mx = -INFINITY;
    if (nsteps <= 0) return mx;
    prologue(false, false);
    const Acc zero = Acc{};
    for (int j = 0; j < nsteps; ++j) {
      kmeta(kofs + (j + 3) * P::KSTEP);
#pragma unroll
      for (int h = 0; h < P::NBLK; ++h) {
        Acc sc = qk_block(j, h, zero);
        if (j >= jfull) mask_block(sc, kofs + j * P::KSTEP + h * 32);
        mx = fmaxf(mx, col_max(sc));
      }
      kstore(j + 2);
      kmeta_use();
      kload();  // K step j+3
      __syncthreads();
    }
    return mx;
  };

  // One pass of the tile.  The softmax reference m is fixed for the whole
  // pass: the exact column max of the first block (pass 1) or of all keys
  // (pass 2, m_given).  Scores arrive from the MFMAs as s*log2(e)/sqrt(d) - m,
  // so p = 2^score with no per-step max, compare or rescale.  Any m gives the
  // same normalised result; pass 1 only fails when a later score exceeds m
  // by so much that some block's probability sum passes kPBig (or o or l
  // stop being finite), and then the tile is redone as pass 2, whose
  // probabilities are all <= 1.  Returns false (nothing written) on failure.
  auto attend = [&](auto exact_tag, float m_given) {
    constexpr bool exact = decltype(exact_tag)::value;
    Acc o[P::NDB];  // zeroed after the prologue, which needs the registers
    float l_run = 0.0f;
    bool bad = false;
    const vec<bf16, 2> ones = {(bf16)1.0f, (bf16)1.0f};
    Op pb[2];
    // probabilities of one block -> two bf16 B operands; the running sum adds
    // those bf16 values (the ones the PV product uses)
    auto softmax_block = [&](const Acc& sc) {
      float ls = 0.0f;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = fast_exp2(sc[8 * m + e]);
        pb[m] = Mma<bf16>::pack(pv);
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const vec<bf16, 2> pp = {pb[m][e], pb[m][e + 1]};
          ls = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, ls, false);
        }
      }
      bad |= !(ls <= kPBig);
      l_run += ls;
    };
    // O^T += V^T P^T for block h of V stage `step`: two 16-key groups, the
    // second group's operands read as the first group's multiply issue
    auto pv_block = [&](int step, int h) {
      // keys h*32 + 16m + 8hh .. +7 of row db*32 + col: unit 4h + 2m + hh
      const bf16* vb = lds + P::V_OFF + (step % P::NVB) * P::VBUF + col * P::VLD;
      const int y = hh ^ vswz(col);
      const int u0 = ((4 * h) ^ y) * 8, u1 = ((4 * h + 2) ^ y) * 8;
      Op va[P::NDB];
#pragma unroll
      for (int db = 0; db < P::NDB; ++db)
        va[db] = *reinterpret_cast<const Op*>(vb + db * 32 * P::VLD + u0);
#pragma unroll
      for (int db = 0; db < P::NDB; ++db) {
        o[db] = Mma32::run(va[db], pb[0], o[db]);
        va[db] = *reinterpret_cast<const Op*>(vb + db * 32 * P::VLD + u1);
      }
#pragma unroll
      for (int db = 0; db < P::NDB; ++db) o[db] = Mma32::run(va[db], pb[1], o[db]);
    };

    Acc negm = Acc{};  // stays 0 (m = 0) for an item with no keys
    Acc s_next;
    if (nsteps > 0) {
      prologue(true, !exact);
      float m;
      if constexpr (exact) {
        m = m_given == -INFINITY ? 0.0f : m_given;
#pragma unroll
        for (int v = 0; v < 16; ++v) negm[v] = -m;
        s_next = qk_block(0, 0, negm);
      } else {
        s_next = qk_block(0, 0, Acc{});
        Acc t = s_next;
        if (jfull == 0) mask_block(t, kofs);
        const float mx = col_max(t);
        m = mx == -INFINITY ? 0.0f : mx;  // a column with no visible key keeps 0
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          negm[v] = -m;
          s_next[v] -= m;
        }
      }
    }

#pragma unroll
    for (int db = 0; db < P::NDB; ++db) o[db] = Acc{};

    // step j: blocks (j, 0) .. (j, NBLK-1), the scores of each next block
    // computed before the current block is exponentiated and multiplied by V.
    // Stages K j+2 and V j+1.
    auto step = [&](int j, auto mask_tag) {
      constexpr bool MASKED = decltype(mask_tag)::value;
      const int kb = kofs + j * P::KSTEP;
      vmeta_use();
      vmeta(kb + 2 * P::KSTEP);
      kmeta(kb + 3 * P::KSTEP);
      vdma(j + 1);  // V step j+1
      // keep the loads at the top of the step: they have the whole step to land
      __builtin_amdgcn_sched_barrier(0);

#pragma unroll
      for (int h = 0; h < P::NBLK; ++h) {
        Acc s_cur = s_next;
        if constexpr (MASKED) mask_block(s_cur, kb + 32 * h);
        s_next = h + 1 < P::NBLK ? qk_block(j, h + 1, negm) : qk_block(j + 1, 0, negm);
        softmax_block(s_cur);
        pv_block(j, h);
      }

      kstore(j + 2);  // K step j+2, loaded during the previous step
      kmeta_use();
      kload();  // K step j+3 (past the end: valid slots, never used)
      // V step j+1 has landed: after its direct loads came one K step's
      // data, still in flight
      vm_wait_n<kDataLoads>();
      vfix(j + 1);
      __syncthreads();
    };
    for (int j = 0; j < jfull; ++j) step(j, std::false_type{});
    for (int j = jfull; j < nsteps; ++j) step(j, std::true_type{});

    const float l_tot = l_run + __shfl_xor(l_run, 32);
    bad |= !(l_tot < INFINITY);
#pragma unroll
    for (int db = 0; db < P::NDB; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) bad |= !(fabsf(o[db][v]) < INFINITY);
    if (!exact && __syncthreads_or(bad && valid)) return false;
    if (!valid) return true;
    if (nsplit > 1) {  // partial of one key chunk: (m, l), and o / l unless empty
      const size_t prow = (size_t)pslot * kPrefillTileRows + wave * 32 + col;
      if (hh == 0) a.pf_ml[prow] = make_float2(-negm[0], l_tot);
      if (l_tot > 0.0f) {
        const float inv = 1.0f / l_tot;
        float* po = a.pf_o + prow * D;
#pragma unroll
        for (int db = 0; db < P::NDB; ++db)
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4)
            *reinterpret_cast<f32x4*>(po + db * 32 + 8 * v4 + 4 * hh) =
                f32x4{o[db][4 * v4] * inv, o[db][4 * v4 + 1] * inv, o[db][4 * v4 + 2] * inv,
                      o[db][4 * v4 + 3] * inv};
      }
      return true;
    }
    const float inv = 1.0f / l_tot;
    bf16* out = (bf16*)a.out + (((size_t)q0 + tok) * a.hq + g * G + head) * D;
#pragma unroll
    for (int db = 0; db < P::NDB; ++db)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        vec<bf16, 4> w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = (bf16)(o[db][4 * v4 + i] * inv);
        *reinterpret_cast<vec<bf16, 4>*>(out + db * 32 + 8 * v4 + 4 * hh) = w;
      }
    return true;
  };

  if (!attend(std::false_type{}, 0.0f)) {
    const float m = row_max();
    attend(std::true_type{}, m);
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
// Inverse of xcd_logical: dispatch position of logical item l (l < n < 2^31,
// so 32-bit arithmetic).
__device__ __forceinline__ unsigned xcd_position(unsigned l, unsigned n) {
  const unsigned q = n / 8, rem = n % 8;
  unsigned x, k;
  if (l < rem * (q + 1)) {
    x = l / (q + 1);
    k = l % (q + 1);
  } else {
    x = rem + (l - rem * (q + 1)) / q;
    k = (l - rem * (q + 1)) % q;
  }
  return k * 8 + x;
}
// xcd_position for one list length n, its two divisions by the per-XCD
// quotient done by multiplication: for a divisor d >= 1 and
// m = floor((2^32 - 1) / d), umulhi(l, m) is floor(l / d) or one less for
// every l < 2^32, and one compare fixes it.
struct XcdMap {
  unsigned q, rem, m1, m0;  // n / 8, n % 8, multipliers for q + 1 and q
  __device__ explicit XcdMap(unsigned n)
      : q(n / 8), rem(n % 8), m1(0xffffffffu / (n / 8 + 1)), m0(n >= 8 ? 0xffffffffu / (n / 8) : 0u) {}
  __device__ static unsigned div(unsigned l, unsigned d, unsigned m, unsigned& r) {
    unsigned x = __umulhi(l, m);
    r = l - x * d;
    if (r >= d) {
      ++x;
      r -= d;
    }
    return x;
  }
  __device__ unsigned position(unsigned l) const {
    const unsigned head = rem * (q + 1);
    unsigned x, k;
    if (l < head) x = div(l, q + 1, m1, k);
    else x = rem + div(l - head, q, m0, k);  // q >= 1 here: l < n
    return k * 8 + x;
  }
};

// Keys of a prefill tile that takes about as long as one decode chunk of the
// mixed launch (8 kv heads, about kSplitTarget keys): measured 61 us per
// chunk against 2.3 us per 64-key step of a tile.
constexpr int kDecodeTileKeys = 4 * kSplitTarget;

// Key-count bucket of a prefill tile (64-key units, capped): the mixed
// launch dispatches the tiles that see more keys first, so the longest tiles
// never start last and leave the rest of the GPU idle at the end.
__device__ __forceinline__ int len_bucket(int L) { return min(max(L, 0) >> 6, 1023); }
// Keys tile k of a request (q_len ql, seq_len L) sees: the slots up to the
// causal limit of its last query row (rows query rows per tile, group heads
// per token), as the tile kernels bound their key loop.  k * rows is below
// ql * group < 2^31, so the row index fits 32 unsigned bits.
__device__ __forceinline__ int tile_keys(int L, int ql, int k, int rows, int group) {
  const int last_tok =
      min((int)(((unsigned)k * (unsigned)rows + (unsigned)rows - 1u) / (unsigned)group), ql - 1);
  return min(L, L - ql + last_tok + 1);
}

// Steps of K/V loads each decode wave keeps in flight.  Measured on MI355X:
// two steps at two workgroups per compute unit (8 waves, 230 VGPRs) beat one
// step at three (12 waves, 159 VGPRs) by about 2% on the 64 x 4097-key
// batches; deeper rings at one workgroup per unit were slower.
constexpr int kDecodeDepth = 2;

// Decode-only launch: logical item = (chunk s, request r, head group hg),
// head group fastest, then request: the workgroups that read the same table
// rows (the same key positions) run on one XCD and share its L2.
// APPEND: each request's new token is written by the workgroups of its last
// chunk (decode_item).
template <typename T, int D, bool ROT, bool APPEND = false>
__global__ void __launch_bounds__(kThreads, 2) decode_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16)))
  unsigned char smem[sizeof(DecodeSmem<T, D, kDecodeDepth + 1, 2>)];
  __shared__ __attribute__((aligned(16))) T s_new[APPEND ? 2 * kWaves * D : 1];
  __shared__ __attribute__((aligned(16))) float s_stash[kWaves * kStashGroup * (D + 2)];
  const long long n = (long long)gridDim.x;
  const long long l = xcd_logical(blockIdx.x, n);
  const int hg = (int)(l % a.nhg);
  const long long rs = l / a.nhg;
  const int r = (int)(rs % a.num_reqs);
  const int p = (int)(rs / a.num_reqs);  // item p: chunks p * dec_cpi ..
  decode_item<T, D, kDecodeDepth, kWaves, ROT, APPEND, 2>(a, r, hg, p * a.dec_cpi, r, smem, s_new,
                                                          a.dec_cpi,
                                                          sizeof(T) == 2 ? s_stash : nullptr);
}

// ---------------------------------------------------------------------------
// shared-span decode: planner and launch
// ---------------------------------------------------------------------------

// 32-bit finaliser of MurmurHash3 (Appleby): spreads a block id's bits so
// that the low bits decide cut candidates independently of how ids were
// allocated.
__device__ __forceinline__ unsigned cdc_mix(unsigned x) {
  x ^= x >> 16;
  x *= 0x85ebca6bu;
  x ^= x >> 13;
  x *= 0xc2b2ae35u;
  x ^= x >> 16;
  return x;
}

__device__ __forceinline__ bool bit_of(const unsigned* w, int b) { return (w[b >> 5] >> (b & 31)) & 1u; }

// Exclusive scan of one int per thread across a workgroup of NT threads
// (NT / 64 waves, at most 64); tot gets the total.
template <int NT>
__device__ __forceinline__ int wg_exclusive_scan(int v, int* s_w, int& tot) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_w[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int t = lane < NT / 64 ? s_w[lane] : 0;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(t, o);
      if (lane >= o) t += y;
    }
    if (lane < NT / 64) s_w[64 + lane] = t;
  }
  __syncthreads();
  tot = s_w[64 + NT / 64 - 1];
  const int before = wave > 0 ? s_w[64 + wave - 1] : 0;
  __syncthreads();
  return before + x - v;
}

// One workgroup per request: the request's chunk start blocks.  Block b > 0
// is a cut when its id is a candidate and none of the kCdcMinGap - 1 blocks
// before it is one; so the cuts inside a span depend only on the span's own
// blocks (past its first kCdcMinGap - 1), whatever precedes it.  Gaps longer
// than kCdcMaxGap blocks are split into equal parts.  Writes cdc_count[r]
// and cdc_start[r][0 .. count] (the last entry is the block count).
__global__ void __launch_bounds__(1024) cdc_chunk_kernel(AttnArgs a, int* cdc_count,
                                                         int* cdc_start) {
  constexpr int NT = 1024;
  constexpr int NW = kCdcMaxBlocks / 32;
  __shared__ unsigned s_cand[NW];
  __shared__ unsigned s_cut[NW];
  __shared__ int s_pos[kCdcMaxBlocks / kCdcMinGap + 3];  // start, cuts (at most (nb - 2) / gap + 1), end
  __shared__ int s_w[128];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = blockIdx.x;
  const int L = seq_len_of(a, r);
  const int nb = min(cdiv(max(L, 0), kBlockSize), kCdcMaxBlocks);
  int* start = cdc_start + (size_t)r * (a.s_max + 1);
  if (nb <= 1) {
    if (tid == 0) {
      cdc_count[r] = 1;
      start[0] = 0;
      start[1] = nb;
    }
    return;
  }
  const int32_t* bt = a.block_table + (size_t)r * a.bt_stride;
  const int nw = cdiv(nb, 32);
  // candidates: each wave takes 4 x 64 consecutive blocks at a time (coalesced
  // ids, four loads in flight per lane)
  for (int b0 = wave * 256; b0 < nb; b0 += NT * 4) {
    int id[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int b = b0 + u * 64 + lane;
      id[u] = b < nb ? bt[b] : 0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int bu = b0 + u * 64;
      const bool c = bu + lane < nb && (cdc_mix((unsigned)id[u]) & kCdcCandMask) == 0;
      const unsigned long long m = __ballot(c);
      if (lane == 0 && bu < nb) {
        s_cand[bu >> 5] = (unsigned)m;
        if ((bu >> 5) + 1 < NW) s_cand[(bu >> 5) + 1] = (unsigned)(m >> 32);
      }
    }
  }
  __syncthreads();
  for (int b0 = wave * 64; b0 < nb; b0 += NT) {
    const int b = b0 + lane;
    bool c = b >= 1 && b < nb && bit_of(s_cand, b);
    for (int k = 1; k < kCdcMinGap; ++k) c = c && (b - k < 0 || !bit_of(s_cand, b - k));
    const unsigned long long m = __ballot(c);
    if (lane == 0) {
      s_cut[b0 >> 5] = (unsigned)m;
      if ((b0 >> 5) + 1 < NW) s_cut[(b0 >> 5) + 1] = (unsigned)(m >> 32);
    }
  }
  __syncthreads();
  // cut positions in order: thread t owns words [t*per, (t+1)*per)
  const int per = cdiv(nw, NT);
  const int w0 = min(nw, tid * per), w1 = min(nw, w0 + per);
  int cnt = 0;
  for (int w = w0; w < w1; ++w) cnt += __popc(s_cut[w]);
  int ncut;
  int k = 1 + wg_exclusive_scan<NT>(cnt, s_w, ncut);
  for (int w = w0; w < w1; ++w) {
    unsigned bits = s_cut[w];
    while (bits) {
      s_pos[k++] = w * 32 + (__ffs(bits) - 1);
      bits &= bits - 1;
    }
  }
  if (tid == 0) {
    s_pos[0] = 0;
    s_pos[ncut + 1] = nb;
  }
  __syncthreads();
  // gaps between consecutive boundaries -> chunks (long gaps in equal parts)
  const int ng = ncut + 1;
  const int gper = cdiv(ng, NT);
  const int g0 = min(ng, tid * gper), g1 = min(ng, g0 + gper);
  int parts = 0;
  for (int gi = g0; gi < g1; ++gi) {
    const int gap = s_pos[gi + 1] - s_pos[gi];
    parts += gap > kCdcMaxGap ? cdiv(gap, kCdcSplitGap) : 1;
  }
  int S;
  int c = wg_exclusive_scan<NT>(parts, s_w, S);
  for (int gi = g0; gi < g1; ++gi) {
    const int b0 = s_pos[gi], gap = s_pos[gi + 1] - b0;
    const int n = gap > kCdcMaxGap ? cdiv(gap, kCdcSplitGap) : 1;
    for (int p = 0; p < n; ++p, ++c)
      if (c < a.s_max) start[c] = b0 + (int)((long long)p * gap / n);
  }
  if (tid == 0) {
    cdc_count[r] = min(S, a.s_max);
    start[min(S, a.s_max)] = nb;
  }
}

// One workgroup: the work list of the shared-span decode.  A chunk whose first
// physical block starts another chunk of the batch too (the same span at the
// same place in several requests) is grouped with those chunks by a hash of
// that block; the other chunks follow, ordered by their first key index, as
// the uniform decode orders its chunks (requests' keys at similar positions
// share cos/sin table rows).  Position i of the list (kv-head group
// innermost) is dispatched where the XCD-contiguous mapping puts logical item
// i, so a group's chunks run side by side on one XCD and the later ones read
// the span from that XCD's L2.  With more than kCdcSortMax chunks the list
// stays in request order.  coff: int[num_reqs + 1] scratch.
__global__ void __launch_bounds__(1024) cdc_order_kernel(AttnArgs a, const int* cdc_count,
                                                         const int* cdc_start, int* coff,
                                                         int4* items, int* nitems) {
  constexpr int NT = 1024;
  constexpr int NH = kCdcSortMax + kCdcPosBuckets;
  __shared__ int s_w[128];
  __shared__ int s_req[kCdcSortMax];  // chunk -> request
  __shared__ int s_key[kCdcSortMax];  // chunk -> hash bucket, then final bucket
  __shared__ int s_hist[NH];
  const int tid = threadIdx.x;
  const int R = a.num_reqs;
  int carry = 0;
  for (int base = 0; base < R; base += NT) {
    const int r = base + tid;
    const int v = r < R ? min(max(cdc_count[r], 1), a.s_max) : 0;
    int tot;
    const int ex = wg_exclusive_scan<NT>(v, s_w, tot);
    if (r < R) coff[r] = carry + ex;
    carry += tot;
  }
  const int C = carry;
  const long long total = (long long)C * a.nhg;
  if (tid == 0) {
    coff[R] = C;
    *nitems = (int)total;
  }
  __syncthreads();
  auto emit = [&](int r, int sc, int pos) {
    for (int hg = 0; hg < a.nhg; ++hg) {
      const unsigned l = (unsigned)((long long)pos * a.nhg + hg);
      items[xcd_position(l, (unsigned)total)] = make_int4(kItemDecode, r, hg, sc);
    }
  };
  // request of chunk x: the last r with coff[r] <= x
  auto locate = [&](int x) {
    int lo = 0, hi = R - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (coff[mid] <= x) lo = mid;
      else hi = mid - 1;
    }
    return lo;
  };
  if (C > kCdcSortMax) {  // request order
    for (int x = tid; x < C; x += NT) {
      const int r = locate(x);
      emit(r, x - coff[r], x);
    }
    return;
  }
  int nbk = 1;
  while (nbk < C) nbk <<= 1;
  for (int i = tid; i < NH; i += NT) s_hist[i] = 0;
  __syncthreads();
  auto first_block = [&](int r, int sc) { return cdc_start[(size_t)r * (a.s_max + 1) + sc]; };
  for (int x = tid; x < C; x += NT) {
    const int r = locate(x);
    const int blk = a.block_table[(size_t)r * a.bt_stride + first_block(r, x - coff[r])];
    const int hb = (int)(cdc_mix((unsigned)blk * 0x9e3779b9u) & (unsigned)(nbk - 1));
    s_req[x] = r;
    s_key[x] = hb;
    atomicAdd(&s_hist[hb], 1);
  }
  __syncthreads();
  // final bucket: the hash bucket when it holds two chunks or more, else a
  // class of the chunk's first block after all hash buckets
  for (int x = tid; x < C; x += NT) {
    const int r = s_req[x];
    const int hb = s_key[x];
    s_key[x] = s_hist[hb] >= 2
                   ? hb
                   : kCdcSortMax + min(first_block(r, x - coff[r]) >> 3, kCdcPosBuckets - 1);
  }
  __syncthreads();
  for (int i = tid; i < NH; i += NT) s_hist[i] = 0;
  __syncthreads();
  for (int x = tid; x < C; x += NT) atomicAdd(&s_hist[s_key[x]], 1);
  __syncthreads();
  // exclusive scan of the histogram: thread t owns buckets [t*per, (t+1)*per)
  constexpr int per = NH / NT;
  int sum = 0;
  for (int i = tid * per; i < (tid + 1) * per; ++i) sum += s_hist[i];
  int tot;
  int run = wg_exclusive_scan<NT>(sum, s_w, tot);
  for (int i = tid * per; i < (tid + 1) * per; ++i) {
    const int v = s_hist[i];
    s_hist[i] = run;
    run += v;
  }
  __syncthreads();
  for (int x = tid; x < C; x += NT) {
    const int r = s_req[x];
    emit(r, x - coff[r], atomicAdd(&s_hist[s_key[x]], 1));
  }
}

// The shared-span decode's main kernel: one work-list item per workgroup.
template <typename T, int D>
__global__ void __launch_bounds__(kThreads, 2) decode_shared_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16)))
  unsigned char smem[sizeof(DecodeSmem<T, D, kDecodeDepth + 1>)];
  if ((int)blockIdx.x >= *a.nitems) return;
  const int4 it = a.items[blockIdx.x];
  decode_item<T, D, kDecodeDepth, kWaves, true>(a, it.y, it.z, it.w, it.y, smem);
}

// Waves per workgroup of the mixed launch.  bf16: eight, so a prefill tile
// holds 256 query rows and each staged (rotated) K step feeds twice the MFMA
// work of a four-wave tile; a decode item then covers eight kv heads.  fp32
// keeps four-wave workgroups.
constexpr int kMixedWavesBf16 = 8;
// Keys per staged step of the bf16 prefill tile.  (Measured alternative:
// four-wave workgroups with 32-key steps fit two workgroups per CU in 80 KB of
// LDS each, so prefill tiles and decode chunks can share a CU; it was slower
// on both the chunked prefill (454 vs 385 us) and the mixed batch (1395 vs
// 1316 us).)
constexpr int kPrefillStep = 64;

template <typename T>
constexpr int mixed_waves() {
  return sizeof(T) == 2 ? kMixedWavesBf16 : kWaves;
}

// Steps of K/V loads each decode wave of the bf16 mixed launch keeps in
// flight.  That launch holds one workgroup of 8 waves per compute unit (the
// prefill tile's LDS and registers); like the decode launch's two 4-wave
// workgroups, its waves keep two steps each in flight.
template <typename T>
constexpr int mixed_decode_depth() {
  return sizeof(T) == 2 ? 2 : 1;
}

template <typename T, int D>
constexpr int prefill_rows() {
  return sizeof(T) == 2 ? Pf<D, mixed_waves<T>(), kPrefillStep>::ROWS : kPrefillRows;
}

template <typename T, int D>
struct MixedSmem {
  static constexpr int PB =
      sizeof(T) == 2 ? Pf<D, mixed_waves<T>(), kPrefillStep>::BYTES : PrefillSmem<T, D>::BYTES;
  static constexpr int DB = (int)sizeof(DecodeSmem<T, D, mixed_decode_depth<T>() + 1>);
  static constexpr int BYTES = PB > DB ? PB : DB;
};

// Mixed launch over the planner's work list.
template <typename T, int D, bool ROT>
__global__ void __launch_bounds__(64 * mixed_waves<T>(), 8 / mixed_waves<T>())
    mixed_kernel(AttnArgs a) {
  constexpr int NW = mixed_waves<T>();
  __shared__ __attribute__((aligned(16))) unsigned char smem[MixedSmem<T, D>::BYTES];
  if ((int)blockIdx.x >= *a.nitems) return;
  const int4 it = a.items[blockIdx.x];
  if (item_kind(it.x) == kItemPrefill) {
    if constexpr (sizeof(T) == 2) {
      prefill_tile_bf16<D, NW, kPrefillStep, ROT>(a, it.y, it.z, it.w, item_split(it.x),
                                                  item_nsplit(it.x), (int)blockIdx.x, smem);
    } else {
      static_assert(ROT, "fp32 prefill tiles always rotate");
      prefill_tile<T, D>(a, it.y, it.z, it.w, smem);
    }
  } else {
    decode_item<T, D, mixed_decode_depth<T>(), NW, ROT>(a, it.y, it.z, it.w,
                                                       (long long)a.cu_q[it.y], smem);
  }
}

// Planner: one workgroup of 1024 threads turns (cu_seqlens_q, seq_lens) into
// the work list, longest items first so that the items that start last are
// short and the compute units run out of work nearly together: the prefill
// tiles that see at least kDecodeTileKeys keys, then the chunks of
// q_len == 1 requests (a decode chunk of about kSplitTarget keys takes about
// as long as a tile over kDecodeTileKeys keys), then the shorter tiles.  A
// launch that splits tiles keeps all prefill items first (a split item's
// partial slot is its list position, below kSplitCUs).  (A workgroup of
// either kind fills a compute unit's LDS and registers, so the two kinds
// cannot share one; interleaving them evenly measured 3% slower on the mixed
// 16-prefill + 128-decode batch.)
// Prefill tiles are ordered longest first by the keys each tile sees, over
// all requests (buckets of 64 keys; ranks inside a bucket from LDS atomics),
// the kv heads (and key chunks) of one tile next to each other, and item i
// is dispatched as workgroup i, so consecutive tiles go to different XCDs.
// A tile's time grows with its keys: with the longest first, the items that
// start last are the shortest and the compute units run out of work nearly
// together (ordering whole requests instead left the tiles of equally long
// requests in request order, and some units idle for 12% of a launch).
// With 8 kv heads every tile of one (request, head) still lands on the same
// XCD.
// Decode chunks are ordered chunk-major inside groups of requests with the
// same chunk count (longest group first): chunk s of every request of a
// group, then chunk s + 1, ...  Consecutive items then read the same key
// positions' cos/sin rows, and an XCD's contiguous range of items needs only
// a few chunk levels' table rows in its L2.  (Ranks inside a group are taken
// with LDS atomics, so the dispatch order of equal-length requests may vary
// between calls; no result depends on it.)
// One step of a 64-bit inclusive scan across a wave by DPP: each lane adds
// the value of the lane CTRL selects (nothing where CTRL selects no lane, or
// where the lane's row of 16 is outside ROW_MASK).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ long long dpp_scan_step(long long x) {
  const unsigned long long u = (unsigned long long)x;
  const unsigned lo =
      (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)u, CTRL, ROW_MASK, 0xf, false);
  const unsigned hi = (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)(u >> 32), CTRL,
                                                            ROW_MASK, 0xf, false);
  return (long long)(u + (((unsigned long long)hi << 32) | lo));
}
// Inclusive scan across the 64 lanes of a wave: shifts by 1, 2, 4 and 8
// lanes inside each row of 16, then the last lane of rows 0 and 2 added to
// rows 1 and 3, then lane 31 added to rows 2 and 3.  (Shuffles through
// ds_bpermute made the planner's scans half of its time.)
__device__ __forceinline__ long long wave_scan(long long x) {
  x = dpp_scan_step<0x111, 0xf>(x);  // row_shr:1
  x = dpp_scan_step<0x112, 0xf>(x);  // row_shr:2
  x = dpp_scan_step<0x114, 0xf>(x);  // row_shr:4
  x = dpp_scan_step<0x118, 0xf>(x);  // row_shr:8
  x = dpp_scan_step<0x142, 0xa>(x);  // row_bcast:15, rows 1 and 3
  x = dpp_scan_step<0x143, 0xc>(x);  // row_bcast:31, rows 2 and 3
  return x;
}
// Lane l's 64-bit value, l uniform across the wave.
__device__ __forceinline__ long long read_lane64(long long x, int l) {
  const unsigned long long u = (unsigned long long)x;
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)u, l);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(u >> 32), l);
  return (long long)(((unsigned long long)hi << 32) | lo);
}

// Inclusive scans of NV values per thread across the 1024-thread planner
// workgroup: a DPP scan inside each wave; then in every wave lane l reads
// wave l's total (l < 16, repeated in each row of 16 lanes), a DPP scan
// inside the row sums them, and the wave takes the sum before it and the
// grand total from two lanes.  One barrier.  (Every lane reading all 16
// totals instead cost 1.7 us of LDS return bandwidth.)  s_w: [16][NV]
// scratch, which the caller may write again only after its next barrier.
// Returns each thread's inclusive prefix; tot gets the workgroup totals.
// Called by every thread of the workgroup.
template <int NV>
__device__ __forceinline__ void plan_scan(long long (&x)[NV], long long (*s_w)[NV],
                                          long long (&tot)[NV]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int v = 0; v < NV; ++v) x[v] = wave_scan(x[v]);
  if (lane == 63)
#pragma unroll
    for (int v = 0; v < NV; ++v) s_w[wave][v] = x[v];
  __syncthreads();
  const int wv = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    long long t = s_w[lane & 15][v];
    t = dpp_scan_step<0x111, 0xf>(t);
    t = dpp_scan_step<0x112, 0xf>(t);
    t = dpp_scan_step<0x114, 0xf>(t);
    t = dpp_scan_step<0x118, 0xf>(t);
    if (wv > 0) x[v] += read_lane64(t, wv - 1);
    tot[v] = read_lane64(t, 15);
  }
}

// Request kinds in the planner's per-request record.
constexpr int kPlanNone = 0, kPlanPrefill = 1, kPlanDecode = 2;

__global__ void __launch_bounds__(1024) plan_kernel(const int32_t* __restrict__ cu_q,
                                                    const int32_t* __restrict__ seq_lens,
                                                    int num_reqs, int hkv, int group, int nhg,
                                                    int kstep, int rows, int len_cap,
                                                    long long max_items,
                                                    int4* __restrict__ items,
                                                    int* __restrict__ count,
                                                    int4* __restrict__ pf_tiles,
                                                    int* __restrict__ pf_count) {
  __shared__ long long s_w2[16][2];
  __shared__ long long s_wt[16][1];
  __shared__ long long s_w1[16][1];
  // per request of the current chunk of 1024: {kind, then for a prefill
  // request its tiles, seq_len and q_len; for a decode request its chunks,
  // the logical decode index of its chunk 0 (head group 0), and the index
  // step from one chunk to the next}
  __shared__ int4 s_meta[1024];
  __shared__ int s_pfn;                // split tiles listed so far
  __shared__ int s_bcnt[1024];         // decode requests per chunk count S
  __shared__ int s_brank[1024];        // ranks handed out so far per S
  __shared__ long long s_bbase[1024];  // first decode-list index of group S
  __shared__ int s_bover;              // some request has 1024 or more chunks
  __shared__ unsigned long long s_dcover;  // decode items of those requests
  __shared__ unsigned long long s_ptot[1024];  // prefill items per context-length bucket
  __shared__ int s_prank[1024];        // prefill tiles placed so far per bucket
  __shared__ long long s_pbase[1024];  // first prefill-list index of each bucket
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  s_bcnt[tid] = 0;
  s_brank[tid] = 0;
  s_ptot[tid] = 0;
  s_prank[tid] = 0;
  if (tid == 0) {
    s_bover = 0;
    s_dcover = 0;
    s_pfn = 0;
  }
  // q_len and (capped) seq_len of request base + tid; the first chunk's stay
  // in registers for the later passes
  auto load = [&](int base, int& ql, int& L) {
    const int r = base + tid;
    ql = 0;
    L = 0;
    if (r < num_reqs) {
      ql = cu_q[r + 1] - cu_q[r];
      L = min(seq_lens[r], len_cap);
    }
  };
  int ql0, L0;
  load(0, ql0, L0);
  // pass 1a: prefill tiles before splitting; they decide the split
  long long tl[1] = {ql0 > 1 ? (long long)hkv * cdiv(ql0 * group, rows) : 0};
  for (int r = tid + 1024; r < num_reqs; r += 1024) {
    const int ql = cu_q[r + 1] - cu_q[r];
    if (ql > 1) tl[0] += (long long)hkv * cdiv(ql * group, rows);
  }
  long long ttot[1];
  plan_scan<1>(tl, s_wt, ttot);
  const int split_max =
      pf_tiles && ttot[0] > 0 && ttot[0] < kSplitCUs ? kSplitCUs / (int)ttot[0] : 1;
  // chunks per tile of a prefill request with L keys
  auto nsplit_of = [&](int L) {
    return split_max > 1 ? max(1, min(split_max, L / kPrefillChunkMin)) : 1;
  };
  // pass 1b, per chunk of 1024 requests: decode requests per chunk count;
  // then prefill items per key-count bucket, the waves taking the chunk's
  // requests in turn and their lanes the request's tiles
  for (int base = 0; base < num_reqs; base += 1024) {
    int ql = ql0, L = L0;
    if (base > 0) load(base, ql, L);
    if (ql == 1) {
      const int S = num_splits(L, kstep);
      if (S < 1024) {
        atomicAdd(&s_bcnt[S], 1);
      } else {
        s_bover = 1;
        atomicAdd(&s_dcover, (unsigned long long)nhg * S);
      }
    }
    s_meta[tid] = make_int4(ql > 1 ? kPlanPrefill : kPlanNone, cdiv(max(ql, 0) * group, rows), L,
                            ql);
    __syncthreads();
    const int nr = min(1024, num_reqs - base);
    for (int rr = wave; rr < nr; rr += 16) {
      const int4 m = s_meta[rr];
      if (m.x != kPlanPrefill) continue;
      const unsigned long long n = (unsigned long long)(hkv * nsplit_of(m.z));
      for (int k = lane; k < m.y; k += 64)
        atomicAdd(&s_ptot[len_bucket(tile_keys(m.z, m.w, k, rows, group))], n);
    }
    __syncthreads();
  }
  // the group / bucket bases (longest first: exclusive suffix sums, total
  // minus the inclusive prefix; thread b holds group or bucket b) and the
  // item totals
  long long x[2] = {(long long)s_bcnt[tid] * tid * nhg, (long long)s_ptot[tid]};
  long long tot[2];
  plan_scan<2>(x, s_w2, tot);
  const long long total_pf = tot[1];
  const long long total_dc = tot[0] + (long long)s_dcover;
  const long long total = total_pf + total_dc;
  s_bbase[tid] = tot[0] - x[0];
  s_pbase[tid] = tot[1] - x[1];
  const bool chunk_major = s_bover == 0;
  // the decode items start after the prefill items of buckets bd and above
  // (s_pbase[bd - 1] of them); the buckets below sit behind the decode items
  // (their bases move by low_shift at use)
  constexpr int bd = kDecodeTileKeys / 64;
  static_assert(bd >= 1 && bd < 1024, "decode items sit between two buckets");
  __syncthreads();
  const long long dec_base = split_max > 1 ? total_pf : s_pbase[bd - 1];
  const long long low_shift = split_max > 1 ? 0 : total_dc;
  // More items than the workspace was sized for means the metadata broke a
  // precondition (cu_seqlens_q not ascending, or total_q / max_seq_len too
  // small): run nothing, and raise the flag that makes the merge launch fill
  // every output row of the launch with NaN, so the failure is visible.
  if (total > max_items) {
    if (tid == 0) {
      count[0] = 0;
      count[1] = 1;
      if (pf_count) *pf_count = 0;
    }
    return;
  }
  if (tid == 0) {
    count[0] = (int)total;
    count[1] = 0;
  }
  // (From here on every decode index is below total_dc <= max_items < 2^31.)
  const XcdMap dec_map((unsigned)total_dc);
  // pass 2, per chunk of 1024 requests: decode offsets (chunk-major: rank in
  // the request's group by LDS atomics; else request order, by a scan),
  // prefill ranks by LDS atomics; then the waves take the chunk's requests
  // in turn and their lanes split each request's items
  long long dc_base = 0;
  for (int base = 0; base < num_reqs; base += 1024) {
    int ql = ql0, L = L0;
    if (base > 0) load(base, ql, L);
    const int S = ql == 1 ? num_splits(L, kstep) : 0;
    int4 m = make_int4(kPlanNone, 0, 0, 0);
    if (chunk_major) {
      // item of chunk sc, head group hg: s_bbase[S] + (sc * s_bcnt[S] + rank) * nhg + hg
      if (ql == 1) {
        const int rank = atomicAdd(&s_brank[S], 1);
        m = make_int4(kPlanDecode, S, (int)(s_bbase[S] + (long long)rank * nhg), s_bcnt[S] * nhg);
      }
    } else {
      // request order: the request's items follow those of the requests before it
      long long y[1] = {ql == 1 ? (long long)nhg * S : 0};
      long long ytot[1];
      plan_scan<1>(y, s_w1, ytot);
      if (ql == 1) m = make_int4(kPlanDecode, S, (int)(dc_base + y[0] - (long long)nhg * S), nhg);
      dc_base += ytot[0];
    }
    if (ql > 1) m = make_int4(kPlanPrefill, cdiv(ql * group, rows), L, ql);
    s_meta[tid] = m;
    __syncthreads();
    const int nr = min(1024, num_reqs - base);
    for (int rr = wave; rr < nr; rr += 16) {
      m = s_meta[rr];
      if (m.x == kPlanPrefill) {  // tiles: each at a place in its bucket, kv heads, then chunks
        const int ns = nsplit_of(m.z);
        const int n = hkv * ns;
        const int code0 = item_code(kItemPrefill, 0, ns > 1 ? ns : 0);
        for (int k = lane; k < m.y; k += 64) {
          const int b = len_bucket(tile_keys(m.z, m.w, k, rows, group));
          long long o = s_pbase[b] + (b < bd ? low_shift : 0) + atomicAdd(&s_prank[b], n);
          for (int g = 0; g < hkv; ++g) {
            if (ns > 1) {
              const int slot = atomicAdd(&s_pfn, 1);
              if (slot < kSplitCUs / 2) pf_tiles[slot] = make_int4(base + rr, g, k, (int)o);
            }
            for (int sp = 0; sp < ns; ++sp, ++o)
              items[o] = make_int4(ns > 1 ? item_code(kItemPrefill, sp, ns) : code0, base + rr,
                                   g, k);
          }
        }
      } else if (m.x == kPlanDecode) {  // chunks, per chunk the kv-head groups
        for (int sc = lane; sc < m.y; sc += 64) {
          const unsigned di0 = (unsigned)m.z + (unsigned)sc * (unsigned)m.w;
          for (int hg = 0; hg < nhg; ++hg)
            items[dec_base + dec_map.position(di0 + hg)] =
                make_int4(kItemDecode, base + rr, hg, sc);
        }
      }
    }
    __syncthreads();
  }
  if (tid == 0 && pf_count) *pf_count = min(s_pfn, kSplitCUs / 2);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

// Measurement hook (pic_set_kernel_events): events that the main kernel of
// each attention call made from this host thread records at its start and
// end.  They are handed to the kernel's dispatch (hipExtLaunchKernelGGL),
// which records them from the dispatch's own timestamps, so the stream gets
// no extra packets.  (Separate event records before and after the kernel
// added about 10 us to every decode step.)  Null when unset: a plain launch.
static thread_local hipEvent_t g_ev_before = nullptr, g_ev_after = nullptr;

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
  a.total_q = h.total_q;
  a.hq = h.hq;
  a.hkv = h.hkv;
  a.group = h.hq / h.hkv;
  a.num_blocks = h.num_blocks;
  a.max_seq_len = h.max_seq_len;
  a.s_max = w.s_max;
  a.nhg = w.nhg;
  a.dec_cpi = 1;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)h.head_dim));
  a.out = h.out;
  unsigned char* ws = (unsigned char*)h.workspace;
  a.ws_ml = (float2*)(ws + w.ml_off);
  a.ws_o = (float*)(ws + w.o_off);
  a.items = (const int4*)(ws + w.items_off);
  a.nitems = (const int*)(ws + w.count_off);
  a.new_k = h.new_k;
  a.new_v = h.new_v;
  if (w.pf_split && h.dtype == PIC_BF16) {
    a.pf_ml = (float2*)(ws + w.pf_ml_off);
    a.pf_o = (float*)(ws + w.pf_o_off);
    a.pf_tiles = (int4*)(ws + w.pf_tiles_off);
    a.pf_count = (int*)(ws + w.pf_count_off);
  }
  return a;
}

// all_reqs: blocks for every (request, kv head) even when no request can have
// several chunks (the mixed launch: those blocks also report a refused work
// list).  A batch of few (request, kv head) pairs splits each merge over
// slices of d so that about 256 blocks share the work (4 x 131k-key decodes:
// 32 pairs of 256 chunks each: the merge 16.4 -> 11.6 us).
template <typename T, int D>
static void launch_combine(const AttnArgs& a, hipStream_t s, bool all_reqs,
                           int split_blocks = 0) {
  const int rh = all_reqs || a.s_max > 1 ? a.num_reqs * a.hkv : 0;
  int dsplit = 1;
  while (a.s_max > 1 && dsplit < D / 8 && (long long)rh * dsplit < 256) dsplit *= 2;
  const int dec_blocks = rh * dsplit;
  if (dec_blocks + split_blocks > 0)
    hipLaunchKernelGGL((combine_kernel<T, D>), dim3((unsigned)(dec_blocks + split_blocks)),
                       dim3(kThreads), 0, s, a, dec_blocks, dsplit);
}

constexpr int kMaxDevices = 64;

// Compute units of the current device (queried once per device).
static std::atomic<int> g_cus[kMaxDevices];
static int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int c = g_cus[dev].load(std::memory_order_relaxed);
  if (c <= 0) {
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        c <= 0)
      c = 256;
    g_cus[dev].store(c, std::memory_order_relaxed);
  }
  return c;
}

// Key chunks per work item of a decode launch with `items` single-chunk
// items.  Two consecutive chunks in one workgroup share its start (chunk
// metadata, query load and rotation) and keep its loads flowing across the
// boundary, and each still writes its own partial, so the results do not
// depend on this choice.  A compute unit then runs ceil(items / CUs) chunks
// with one chunk per item and 2 x ceil(items / (2 CUs)) with two: pair when
// that is no more (measured on 16 decode batches of 1-128 requests x 2k-33k
// keys: pairing gains 1.5-4.5% wherever this holds and loses 10-70% on the
// batches where it does not).
static int decode_chunks_per_item(long long items) {
  const long long cus = device_cus();
  const long long one = (items + cus - 1) / cus;
  const long long two = 2 * ((items + 2 * cus - 1) / (2 * cus));
  return two <= one ? 2 : 1;
}

template <typename T, int D, bool ROT>
static int launch_decode(AttnArgs a, hipStream_t s) {
  const long long n1 = (long long)a.num_reqs * a.s_max * a.nhg;
  if (n1 > 0x7fffffffLL || (long long)a.num_reqs * a.hkv > 0x7fffffffLL) return PIC_EUNSUPPORTED;
  a.dec_cpi = a.group <= kStashGroup ? decode_chunks_per_item(n1) : 1;
  const long long n = (long long)a.num_reqs * cdiv(a.s_max, a.dec_cpi) * a.nhg;
  if constexpr (ROT) {
    if (a.new_k) {
      hipExtLaunchKernelGGL((decode_kernel<T, D, true, true>), dim3((unsigned)n),
                            dim3(kThreads), 0, s, g_ev_before, g_ev_after, 0, a);
      launch_combine<T, D>(a, s, false);
      return hipGetLastError() == hipSuccess ? PIC_OK : PIC_EHIP;
    }
  }
  hipExtLaunchKernelGGL((decode_kernel<T, D, ROT>), dim3((unsigned)n), dim3(kThreads), 0, s,
                        g_ev_before, g_ev_after, 0, a);
  launch_combine<T, D>(a, s, false);
  return hipGetLastError() == hipSuccess ? PIC_OK : PIC_EHIP;
}

template <typename T, int D, bool ROT>
static int launch_mixed(const AttnArgs& a, const WorkspaceLayout& w, const AttnHostArgs& h,
                        hipStream_t s) {
  if (w.max_items > 0x7fffffffLL || (long long)h.num_reqs * h.hkv + kSplitCUs > 0x7fffffffLL)
    return PIC_EUNSUPPORTED;
  unsigned char* ws = (unsigned char*)h.workspace;
  const int len_cap = (int)min((long long)h.max_seq_len,
                              (long long)h.block_table_stride * kBlockSize);
  const bool split = a.pf_tiles != nullptr;  // bf16, and the launch may split tiles
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, s, h.cu_seqlens_q, h.seq_lens,
                     h.num_reqs, h.hkv, h.hq / h.hkv, cdiv(h.hkv, mixed_waves<T>()),
                     Cfg<T, D>::KSTEP, prefill_rows<T, D>(), len_cap,
                     w.max_items, (int4*)(ws + w.items_off), (int*)(ws + w.count_off),
                     a.pf_tiles, a.pf_count);
  hipExtLaunchKernelGGL((mixed_kernel<T, D, ROT>), dim3((unsigned)w.max_items),
                        dim3(64 * mixed_waves<T>()), 0, s, g_ev_before, g_ev_after, 0, a);
  // Always launched: whether a request has q_len == 1 is device data, and its
  // blocks exit at once where there is nothing to merge.
  launch_combine<T, D>(a, s, true, split ? kSplitCUs / 2 * kMergeParts : 0);
  return hipGetLastError() == hipSuccess ? PIC_OK : PIC_EHIP;
}

// One decode call: position-free (ROT) or over an already rotated cache.
template <bool ROT>
static int attn_decode(const AttnHostArgs& h, hipStream_t s) {
  int st = check_attn_common(h, ROT, true);
  if (st || h.num_reqs == 0) return st;
  if (!ROT && h.dtype != PIC_BF16) return PIC_EUNSUPPORTED;
  const WorkspaceLayout w = workspace_layout(h.num_reqs, h.num_reqs, h.max_seq_len, h.hq,
                                             h.hkv, h.head_dim, true);
  const AttnArgs a = make_args(h, w);
  if (h.dtype == PIC_BF16)
    return h.head_dim == 128 ? launch_decode<bf16, 128, ROT>(a, s)
                             : launch_decode<bf16, 64, ROT>(a, s);
  if constexpr (ROT) {
    return h.head_dim == 128 ? launch_decode<float, 128, true>(a, s)
                             : launch_decode<float, 64, true>(a, s);
  }
  return PIC_EUNSUPPORTED;
}

// Shared-span decode: chunking, ordering, decode, merge.
template <typename T, int D>
static int launch_decode_shared(const AttnArgs& a, const SharedDecodeLayout& w,
                                const AttnHostArgs& h, hipStream_t s) {
  unsigned char* ws = (unsigned char*)h.workspace;
  int* cnt = (int*)(ws + w.cnt_off);
  int* start = (int*)(ws + w.start_off);
  hipLaunchKernelGGL(cdc_chunk_kernel, dim3((unsigned)h.num_reqs), dim3(1024), 0, s, a, cnt,
                     start);
  hipLaunchKernelGGL(cdc_order_kernel, dim3(1), dim3(1024), 0, s, a, cnt, start,
                     (int*)(ws + w.coff_off), (int4*)(ws + w.items_off),
                     (int*)(ws + w.count_off));
  hipExtLaunchKernelGGL((decode_shared_kernel<T, D>), dim3((unsigned)w.max_items),
                        dim3(kThreads), 0, s, g_ev_before, g_ev_after, 0, a);
  launch_combine<T, D>(a, s, false);
  return hipGetLastError() == hipSuccess ? PIC_OK : PIC_EHIP;
}

static int attn_decode_shared(const AttnHostArgs& h, hipStream_t s) {
  if (h.num_reqs < 0 || h.max_seq_len < 0 || h.hq <= 0 || h.hkv <= 0)
    return check_attn_args(h, true, 0);
  const SharedDecodeLayout w = shared_decode_layout(h.num_reqs, h.max_seq_len, h.hq, h.hkv,
                                                    h.head_dim);
  int st = check_attn_args(h, true, w.total);
  if (st || h.num_reqs == 0) return st;
  if (!w.supported) return PIC_EUNSUPPORTED;
  WorkspaceLayout dl{};
  dl.count_off = w.count_off;
  dl.items_off = w.items_off;
  dl.ml_off = w.ml_off;
  dl.o_off = w.o_off;
  dl.s_max = w.s_max;
  dl.nhg = w.nhg;
  dl.max_items = w.max_items;
  AttnArgs a = make_args(h, dl);
  unsigned char* ws = (unsigned char*)h.workspace;
  a.cdc_count = (const int*)(ws + w.cnt_off);
  a.cdc_start = (const int*)(ws + w.start_off);
  if (h.dtype == PIC_BF16)
    return h.head_dim == 128 ? launch_decode_shared<bf16, 128>(a, w, h, s)
                             : launch_decode_shared<bf16, 64>(a, w, h, s);
  return h.head_dim == 128 ? launch_decode_shared<float, 128>(a, w, h, s)
                           : launch_decode_shared<float, 64>(a, w, h, s);
}

// Scratch of pic_attn_decode_noalloc: the decode workspace (chunk partials)
// in a fixed device array instead of caller memory, for callers that cannot
// allocate.  Each device holds its own copy for the life of the process; its
// address is looked up once per device with that device current (the array's
// name is a host-side stand-in, never a device address).
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
static std::atomic<void*> g_scratch_ptr[kMaxDevices];

static void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

template <bool ROT>
static int attn_prefill(const AttnHostArgs& h, hipStream_t s) {
  int st = check_attn_common(h, ROT, false);
  if (st || h.num_reqs == 0 || h.total_q == 0) return st;
  if (!h.cu_seqlens_q || h.max_q_len < 0) return PIC_EINVAL;
  if (!ROT && h.dtype != PIC_BF16) return PIC_EUNSUPPORTED;
  const WorkspaceLayout w = workspace_layout(h.num_reqs, h.total_q, h.max_seq_len, h.hq, h.hkv,
                                             h.head_dim);
  const AttnArgs a = make_args(h, w);
  if (h.dtype == PIC_BF16)
    return h.head_dim == 128 ? launch_mixed<bf16, 128, ROT>(a, w, h, s)
                             : launch_mixed<bf16, 64, ROT>(a, w, h, s);
  if constexpr (ROT) {
    return h.head_dim == 128 ? launch_mixed<float, 128, true>(a, w, h, s)
                             : launch_mixed<float, 64, true>(a, w, h, s);
  }
  return PIC_EUNSUPPORTED;
}

}  // namespace pic

using pic::AttnHostArgs;

extern "C" int pic_set_kernel_events(void* before, void* after) {
  if ((before == nullptr) != (after == nullptr)) return PIC_EINVAL;
  pic::g_ev_before = (hipEvent_t)before;
  pic::g_ev_after = (hipEvent_t)after;
  return PIC_OK;
}

// Timing events: HIP events without the system-scope acquire / release that a
// default event record carries (hipEventDisableSystemFence).  That fence
// writes back and invalidates caches at every record and slows the work that
// follows; these events only measure, nothing reads memory through them.
extern "C" int pic_timing_event_create(void** event) {
  if (!event) return PIC_EINVAL;
  *event = nullptr;
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return PIC_EHIP;
  // recorded once on the default stream, so a pair never recorded since reads 0 ms
  if (hipEventRecord(e, nullptr) != hipSuccess) {
    hipEventDestroy(e);
    return PIC_EHIP;
  }
  *event = e;
  return PIC_OK;
}

extern "C" int pic_timing_event_record(void* event, void* stream) {
  if (!event) return PIC_EINVAL;
  return hipEventRecord((hipEvent_t)event, (hipStream_t)stream) == hipSuccess ? PIC_OK : PIC_EHIP;
}

extern "C" int pic_timing_event_elapsed_ms(void* start, void* stop, float* ms) {
  if (!start || !stop || !ms) return PIC_EINVAL;
  return hipEventElapsedTime(ms, (hipEvent_t)start, (hipEvent_t)stop) == hipSuccess ? PIC_OK
                                                                                    : PIC_EHIP;
}

extern "C" int pic_timing_event_destroy(void* event) {
  if (!event) return PIC_OK;
  return hipEventDestroy((hipEvent_t)event) == hipSuccess ? PIC_OK : PIC_EHIP;
}

extern "C" int pic_attn_decode(const void* q, const int32_t* q_pos, const void* k_pool,
                               const void* v_pool, const int32_t* block_table,
                               int block_table_stride, const int32_t* seq_lens,
                               const int32_t* cu_seqlens_k, const int32_t* k_pos,
                               const float* cos_tab, const float* sin_tab, int max_pos,
                               int num_reqs, int num_q_heads, int num_kv_heads, int head_dim,
                               int block_size, int num_blocks, int max_seq_len, int dtype,
                               void* out, void* workspace, size_t workspace_bytes,
                               void* stream) {
  const AttnHostArgs h{q, nullptr, q_pos, k_pool, v_pool, block_table, block_table_stride,
                       seq_lens, cu_seqlens_k, k_pos, cos_tab, sin_tab, max_pos, num_reqs,
                       num_reqs, 1, num_q_heads, num_kv_heads, head_dim, block_size,
                       num_blocks, max_seq_len, dtype, out, workspace, workspace_bytes};
  return pic::attn_decode<true>(h, (hipStream_t)stream);
}

extern "C" int pic_attn_decode_append(const void* q, const void* new_k, const void* new_v,
                                      const int32_t* q_pos, const void* k_pool, const void* v_pool,
                                      const int32_t* block_table, int block_table_stride,
                                      const int32_t* seq_lens, const int32_t* cu_seqlens_k,
                                      const int32_t* k_pos, const float* cos_tab,
                                      const float* sin_tab, int max_pos, int num_reqs,
                                      int num_q_heads, int num_kv_heads, int head_dim,
                                      int block_size, int num_blocks, int max_seq_len, int dtype,
                                      void* out, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  AttnHostArgs h{q, nullptr, q_pos, k_pool, v_pool, block_table, block_table_stride,
                 seq_lens, cu_seqlens_k, k_pos, cos_tab, sin_tab, max_pos, num_reqs,
                 num_reqs, 1, num_q_heads, num_kv_heads, head_dim, block_size,
                 num_blocks, max_seq_len, dtype, out, workspace, workspace_bytes};
  if (num_reqs > 0 && (!new_k || !new_v)) return PIC_EINVAL;
  h.new_k = new_k;
  h.new_v = new_v;
  return pic::attn_decode<true>(h, (hipStream_t)stream);
}

extern "C" int pic_attn_decode_noalloc(const void* q, const int32_t* q_pos, const void* k_pool,
                                       const void* v_pool, const int32_t* block_table,
                                       int block_table_stride, const int32_t* seq_lens,
                                       const int32_t* cu_seqlens_k, const int32_t* k_pos,
                                       const float* cos_tab, const float* sin_tab, int max_pos,
                                       int num_reqs, int num_q_heads, int num_kv_heads,
                                       int head_dim, int block_size, int num_blocks,
                                       int max_seq_len, int dtype, void* out, void* stream) {
  void* ws = pic::scratch_address();
  if (!ws) return PIC_EHIP;
  const AttnHostArgs h{q, nullptr, q_pos, k_pool, v_pool, block_table, block_table_stride,
                       seq_lens, cu_seqlens_k, k_pos, cos_tab, sin_tab, max_pos, num_reqs,
                       num_reqs, 1, num_q_heads, num_kv_heads, head_dim, block_size,
                       num_blocks, max_seq_len, dtype, out, ws, pic::kNoAllocScratchBytes};
  return pic::attn_decode<true>(h, (hipStream_t)stream);
}

extern "C" int pic_attn_decode_shared(const void* q, const int32_t* q_pos, const void* k_pool,
                                      const void* v_pool, const int32_t* block_table,
                                      int block_table_stride, const int32_t* seq_lens,
                                      const int32_t* cu_seqlens_k, const int32_t* k_pos,
                                      const float* cos_tab, const float* sin_tab, int max_pos,
                                      int num_reqs, int num_q_heads, int num_kv_heads,
                                      int head_dim, int block_size, int num_blocks,
                                      int max_seq_len, int dtype, void* out, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  const AttnHostArgs h{q, nullptr, q_pos, k_pool, v_pool, block_table, block_table_stride,
                       seq_lens, cu_seqlens_k, k_pos, cos_tab, sin_tab, max_pos, num_reqs,
                       num_reqs, 1, num_q_heads, num_kv_heads, head_dim, block_size,
                       num_blocks, max_seq_len, dtype, out, workspace, workspace_bytes};
  return pic::attn_decode_shared(h, (hipStream_t)stream);
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
  const AttnHostArgs h{q, cu_seqlens_q, q_pos, k_pool, v_pool, block_table, block_table_stride,
                       seq_lens, cu_seqlens_k, k_pos, cos_tab, sin_tab, max_pos, num_reqs,
                       total_q, max_q_len, num_q_heads, num_kv_heads, head_dim, block_size,
                       num_blocks, max_seq_len, dtype, out, workspace, workspace_bytes};
  return pic::attn_prefill<true>(h, (hipStream_t)stream);
}

extern "C" int pic_attn_decode_rotated(const void* q, const int32_t* q_pos, const void* k_pool,
                                       const void* v_pool, const int32_t* block_table,
                                       int block_table_stride, const int32_t* seq_lens,
                                       const float* cos_tab, const float* sin_tab, int max_pos,
                                       int num_reqs, int num_q_heads, int num_kv_heads,
                                       int head_dim, int block_size, int num_blocks,
                                       int max_seq_len, int dtype, void* out, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  const AttnHostArgs h{q, nullptr, q_pos, k_pool, v_pool, block_table, block_table_stride,
                       seq_lens, nullptr, nullptr, cos_tab, sin_tab, max_pos, num_reqs,
                       num_reqs, 1, num_q_heads, num_kv_heads, head_dim, block_size,
                       num_blocks, max_seq_len, dtype, out, workspace, workspace_bytes};
  return pic::attn_decode<false>(h, (hipStream_t)stream);
}

extern "C" int pic_attn_prefill_rotated(const void* q, const int32_t* cu_seqlens_q,
                                        const int32_t* q_pos, const void* k_pool,
                                        const void* v_pool, const int32_t* block_table,
                                        int block_table_stride, const int32_t* seq_lens,
                                        const float* cos_tab, const float* sin_tab,
                                        int max_pos, int num_reqs, int total_q, int max_q_len,
                                        int num_q_heads, int num_kv_heads, int head_dim,
                                        int block_size, int num_blocks, int max_seq_len,
                                        int dtype, void* out, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  const AttnHostArgs h{q, cu_seqlens_q, q_pos, k_pool, v_pool, block_table, block_table_stride,
                       seq_lens, nullptr, nullptr, cos_tab, sin_tab, max_pos, num_reqs,
                       total_q, max_q_len, num_q_heads, num_kv_heads, head_dim, block_size,
                       num_blocks, max_seq_len, dtype, out, workspace, workspace_bytes};
  return pic::attn_prefill<false>(h, (hipStream_t)stream);
}
