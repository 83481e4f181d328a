// sv_accept.hpp -- row statistics, the acceptance rules and the correction/bonus
// sampler of the verify step (gfx950).
//
// Greedy rule ([MTP-drafters] 3.2, [Self-spec] 3.1): accept draft i while it equals
// the argmax of slot i; the first mismatch ends the round with the slot's argmax;
// all accepted gives slot gamma's argmax as the bonus ([Infra-ch8] "where the extra
// token comes from").
// Sampling rule ([MTP-deep-dive] 2.2, [Infra-ch8] "why the output does not change",
// [Self-spec] 3.2): accept draft x with probability min(1, p(x)/q(x)), tested as
// u * q(x) < p(x) with a 24-bit Philox uniform per (sequence, position); the first
// rejected slot draws from max(0, p - q) (from p when that is zero everywhere);
// all accepted draws the bonus from p_gamma.  Draws use Gumbel-max over Philox noise
// keyed by (seed, sequence, position, vocab entry), so any partition of the vocabulary
// over workgroups gives the same token.
#pragma once

#include "sv_device.hpp"

namespace sv {

// Per-sequence state handed from the accept kernel to the sampler.
struct SeqState {
  int n;          // accepted drafts (-1: invalid sequence)
  float m;        // max logit of slot n
  float z;        // sum of exp2((l - m) * c) over slot n
  int pad;
};

// The state is read by other workgroups of the same launch in the fused sampler:
// written through to the coherent memory side.
__device__ __forceinline__ void store_state(SeqState* p, int n, float m, float z) {
  store_coherent(&p->n, n);
  store_coherent(&p->m, m);
  store_coherent(&p->z, z);
}

// Best (score, index) of a vocabulary chunk for the residual and for p itself.
struct SamplePart {
  float sr;
  int ir;
  float sp;
  int ip;
  int any_r;      // some r_v > 0 in this chunk
  int pad[3];
};

__device__ __forceinline__ void store_spart(SamplePart* p, const SamplePart& v) {
  store_coherent(&p->sr, v.sr);
  store_coherent(&p->ir, v.ir);
  store_coherent(&p->sp, v.sp);
  store_coherent(&p->ip, v.ip);
  store_coherent(&p->any_r, v.any_r);
}


// Row statistics of float32 logits [M, V]: one wavefront per (row, chunk of LCH).
constexpr int LCH = 4096;

__global__ __launch_bounds__(256) void k_stats_logits(const float* __restrict__ logits, RowPart* __restrict__ part,
                                                      int M, int V, float c) {
  const int lane = threadIdx.x & 63;
  const long item = long(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int nch = (V + LCH - 1) / LCH;
  if (item >= long(M) * nch) return;
  const int row = int(item % M), ch = int(item / M);
  const float* l = logits + size_t(row) * V;
  const int v0 = ch * LCH, v1 = min(V, v0 + LCH);
  float m = -INFINITY;
  int am = 0x7fffffff;
  for (int v = v0 + lane; v < v1; v += 64) {
    float x = l[v];
    if (x > m) { m = x; am = v; }           // ascending v per lane: first max kept
  }
  float s = 0.0f;
  if (c != 0.0f && am != 0x7fffffff)
    for (int v = v0 + lane; v < v1; v += 64) s += exp2f((l[v] - m) * c);
  wave_merge_stat(m, s, am, c);
  if (lane == 0) store_part(part + size_t(ch) * M + row, m, s, am);
}

struct AcceptArgs {
  const RowPart* part;    // [P, M]
  int P;
  const float* logits;    // [M, V]
  const float* xlogit;    // [M] or null: logit of each slot's draft token, stored by the product
  const int* draft;       // [B, gamma] (or tokens [B, G1] with draft_stride = G1, offset 1)
  int draft_stride, draft_offset;
  const void* q;          // [B, gamma, V]
  int q_bf16;
  const int64_t* pos0;    // [B]
  const int* invalid;     // [B] or null: 1 = invalid sequence (bad token id / cache overflow)
  int* len;               // [B] or null: cache lengths to advance
  int* n_accepted;        // [B]
  int* tokens_out;        // [B, G1]
  SeqState* state;        // [B] (sampling)
  uint64_t seed;
  int B, gamma, V;
  float c;                // log2(e) / T
  int sample;             // 0 greedy, 1 sampling
};

// Merge the P partials of one row over a wavefront: independent loads, 8 per lane
// in flight, then a shuffle reduction.
__device__ __forceinline__ void merge_row(const RowPart* __restrict__ part, int P, int M, int row, float c, float& m,
                                          float& s, int& am) {
  const int lane = threadIdx.x & 63;
  m = -INFINITY; s = 0.0f; am = 0x7fffffff;
  for (int p0 = lane; p0 < P; p0 += 64 * 8) {
    RowPart rp[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int p = p0 + 64 * u;
      if (p < P) rp[u] = part[size_t(p) * M + row];
      else { rp[u].m = -INFINITY; rp[u].s = 0.0f; rp[u].a = 0x7fffffff; rp[u].pad = 0; }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) merge_stat(m, s, am, rp[u].m, rp[u].s, rp[u].a, c);
  }
  wave_allmerge_stat(m, s, am, c);
}

// Acceptance for sequences [b0, b0 + nb) by one workgroup (of four or more wavefronts).
// Phase 1: the wavefronts merge the statistics partials of the nb * G1 rows
// (row j by wave j % waves); phase 2: wave w applies the rule to sequences b0 + w,
// b0 + w + waves, ... with lane i holding slot i.  Requires nb * G1 <= ACC_MAX_ROWS.
constexpr int ACC_MAX_ROWS = 64;

__device__ __forceinline__ void accept_block(const AcceptArgs& a, int b0, int nb) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G1 = a.gamma + 1;
  const int M = a.B * G1;
  const float cs = a.sample ? a.c : 0.0f;
  __shared__ float s_m[ACC_MAX_ROWS], s_s[ACC_MAX_ROWS];
  __shared__ int s_a[ACC_MAX_ROWS];
  for (int j = wave; j < nb * G1; j += int(blockDim.x >> 6)) {
    float m, s;
    int am;
    merge_row(a.part, a.P, M, b0 * G1 + j, cs, m, s, am);
    if (lane == 0) { s_m[j] = m; s_s[j] = s; s_a[j] = am; }
  }
  __syncthreads();
  for (int bl = wave; bl < nb; bl += int(blockDim.x >> 6)) {
    const int b = b0 + bl;
    float my_m = -INFINITY, my_s = 0.0f;
    int my_a = 0x7fffffff;
    if (lane < G1) { my_m = s_m[bl * G1 + lane]; my_s = s_s[bl * G1 + lane]; my_a = s_a[bl * G1 + lane]; }
    const bool bad = a.invalid && a.invalid[b];
    if (bad) {
      if (lane < G1) a.tokens_out[b * G1 + lane] = -1;
      if (lane == 0) {
        a.n_accepted[b] = -1;
        if (a.sample) store_state(a.state + b, -1, 0.0f, 0.0f);
      }
      continue;
    }
    int x = -1;
    if (lane < a.gamma) x = a.draft[size_t(b) * a.draft_stride + a.draft_offset + lane];
    const bool inr = x >= 0 && x < a.V;
    bool ok;
    if (!a.sample) {
      ok = inr && x == my_a;
    } else {
      float px = 0.0f, qx = 0.0f;
      if (inr) {
        const float l = a.xlogit ? a.xlogit[b * G1 + lane] : a.logits[size_t(b * G1 + lane) * a.V + x];
        px = exp2f((l - my_m) * a.c) / my_s;
        const size_t qi = (size_t(b) * a.gamma + lane) * a.V + x;
        qx = a.q_bf16 ? bf16_to_f32(reinterpret_cast<const bf16_t*>(a.q)[qi]) : reinterpret_cast<const float*>(a.q)[qi];
      }
      const float u = lane < a.gamma ? accept_uniform(a.seed, uint64_t(b), uint64_t(a.pos0[b] + lane + 1)) : 1.0f;
      ok = double(u) * double(qx) < double(px);      // exact: 24-bit u times <= 24-bit q
    }
    const unsigned long long rej = __ballot(lane < a.gamma && !ok);
    const int n = rej ? __ffsll(rej) - 1 : a.gamma;
    const int tok_n = __shfl(my_a, n);
    const float m_n = __shfl(my_m, n), s_n = __shfl(my_s, n);
    if (lane < G1) {
      int t = -1;
      if (lane < n) t = x;
      else if (lane == n && !a.sample) t = tok_n;
      a.tokens_out[b * G1 + lane] = t;
    }
    if (lane == 0) {
      if (!a.sample) {
        a.n_accepted[b] = n;
        if (a.len) a.len[b] += n + 1;
      } else {
        store_state(a.state + b, n, m_n, s_n);
      }
    }
  }
}

// The acceptance as a launch of its own: one workgroup per sequence with a wavefront
// per row of it (at least four), so that every row's partials are merged at once (the
// same merge order, so the same bits, as four wavefronts taking the rows in turn).
__global__ __launch_bounds__(1024) void k_accept(AcceptArgs a) { accept_block(a, blockIdx.x, 1); }

// Ticket of the calling workgroup on a one-shot counter.  Every thread first waits
// for its own stores to complete (the data handed over was written with
// store_coherent, so completion means it reached the coherent memory side); then
// one thread takes a ticket.  The workgroup that draws the last ticket issues an
// acquire fence (its caches may hold stale copies from an earlier launch) and can
// then read the handed-over data with ordinary loads.  It resets the counter for
// the next launch.
__device__ __forceinline__ bool last_workgroup(unsigned* counter, unsigned total) {
  __shared__ unsigned s_ticket;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) s_ticket = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (s_ticket != total - 1) return false;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  if (threadIdx.x == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

struct SampleArgs {
  const float* logits;    // [M, V]
  const void* q;          // [B, gamma, V]
  int q_bf16;
  const int64_t* pos0;
  const SeqState* state;  // [B]
  SamplePart* spart;      // [B, nch]
  uint64_t seed;
  int B, gamma, V, chunk, nch;
  float c;
  unsigned* counter;      // non-null: the last workgroup finishes every sequence
  int* n_accepted;
  int* tokens_out;
  int* len;
};

__device__ __forceinline__ void sample_finish_wave(const SampleArgs& a, int b);

// grid nch * B: Gumbel-max over one chunk of row n_b.  Each thread draws four
// consecutive vocab entries from one Philox block.
__global__ __launch_bounds__(256) void k_sample(SampleArgs a) {
  const int b = int(blockIdx.x / unsigned(a.nch)), ch = int(blockIdx.x % unsigned(a.nch));
  const SeqState st = a.state[b];
  SamplePart out;
  out.sr = -INFINITY; out.ir = 0x7fffffff; out.sp = -INFINITY; out.ip = 0x7fffffff; out.any_r = 0;
  out.pad[0] = out.pad[1] = out.pad[2] = 0;
  if (st.n < 0) {
    if (threadIdx.x == 0) store_spart(a.spart + size_t(b) * a.nch + ch, out);
    if (a.counter && last_workgroup(a.counter, gridDim.x)) {
      for (int bb = threadIdx.x >> 6; bb < a.B; bb += 4) sample_finish_wave(a, bb);
    }
    return;
  }
  const int G1 = a.gamma + 1;
  const bool resid = st.n < a.gamma;
  const float* l = a.logits + size_t(b * G1 + st.n) * a.V;
  const size_t qrow = (size_t(b) * a.gamma + (resid ? st.n : 0)) * a.V;
  const uint64_t pos = uint64_t(a.pos0[b] + st.n + 1);
  const int v0 = ch * a.chunk, v1 = min(a.V, v0 + a.chunk);
  float sr = -INFINITY, sp = -INFINITY;
  int ir = 0x7fffffff, ip = 0x7fffffff, any_r = 0;
  for (int vb = v0 + 4 * threadIdx.x; vb < v1; vb += 4 * blockDim.x) {
    float lv[4], qv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int v = min(vb + e, v1 - 1);
      lv[e] = l[v];
      qv[e] = 0.0f;
      if (resid)
        qv[e] = a.q_bf16 ? bf16_to_f32(reinterpret_cast<const bf16_t*>(a.q)[qrow + v])
                         : reinterpret_cast<const float*>(a.q)[qrow + v];
    }
    const Philox4 w = philox4x64_10(uint64_t(vb) >> 2, pos, uint64_t(b), TAG_GUMBEL, a.seed, 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int v = vb + e;
      if (v >= v1) break;
      const float U = gumbel_uniform_from_word(w.w[e]);
      const float G = -logf(-logf(U));
      const float p = exp2f((lv[e] - st.m) * a.c) / st.z;
      if (p > 0.0f) {
        const float sc = logf(p) + G;
        if (sc > sp) { sp = sc; ip = v; }
      }
      if (resid) {
        const float r = fmaxf(p - qv[e], 0.0f);
        if (r > 0.0f) {
          any_r = 1;
          const float sc = logf(r) + G;
          if (sc > sr) { sr = sc; ir = v; }
        }
      }
    }
  }
  wave_merge_best(sr, ir);
  wave_merge_best(sp, ip);
  any_r = __any(any_r) ? 1 : 0;
  __shared__ float s_sr[4], s_sp[4];
  __shared__ int s_ir[4], s_ip[4], s_any[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) { s_sr[wave] = sr; s_ir[wave] = ir; s_sp[wave] = sp; s_ip[wave] = ip; s_any[wave] = any_r; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 0; w < int(blockDim.x >> 6); ++w) {
      merge_best(out.sr, out.ir, s_sr[w], s_ir[w]);
      merge_best(out.sp, out.ip, s_sp[w], s_ip[w]);
      out.any_r |= s_any[w];
    }
    store_spart(a.spart + size_t(b) * a.nch + ch, out);
  }
  if (a.counter && last_workgroup(a.counter, gridDim.x)) {
    for (int bb = threadIdx.x >> 6; bb < a.B; bb += 4) sample_finish_wave(a, bb);
  }
}

// One wavefront merges the chunk winners of sequence b and writes its last token,
// n and len.  p itself is used where p is drawn from (bonus) or where the residual
// is zero everywhere.
__device__ __forceinline__ void sample_finish_wave(const SampleArgs& a, int b) {
  const int lane = threadIdx.x & 63;
  const SeqState st = a.state[b];
  if (st.n < 0) return;        // invalid: the accept step wrote the outputs
  float sr = -INFINITY, sp = -INFINITY;
  int ir = 0x7fffffff, ip = 0x7fffffff, any_r = 0;
  for (int c = lane; c < a.nch; c += 64) {
    const SamplePart p = a.spart[size_t(b) * a.nch + c];
    merge_best(sr, ir, p.sr, p.ir);
    merge_best(sp, ip, p.sp, p.ip);
    any_r |= p.any_r;
  }
  wave_merge_best(sr, ir);
  wave_merge_best(sp, ip);
  any_r = __any(any_r) ? 1 : 0;
  if (lane == 0) {
    const bool resid = st.n < a.gamma && any_r;
    a.tokens_out[b * (a.gamma + 1) + st.n] = resid ? ir : ip;
    a.n_accepted[b] = st.n;
    if (a.len) a.len[b] += st.n + 1;
  }
}

// One wavefront per sequence (used when the batch is too large to finish in the
// sampler's last workgroup).
__global__ __launch_bounds__(256) void k_sample_finish(SampleArgs a) {
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (b < a.B) sample_finish_wave(a, b);
}

}  // namespace sv
