// tree.hip - greedy verification of draft token trees (the walk of the DDTree
// section of chzhyang, "Speculative Decoding: Medusa, MTP, EAGLE, DFlash,
// DDTree, and DSpark", section 5), all node rows at once or step by step.
#include "sv_common.hpp"

namespace {

// ------------------------------------------------------------------ token trees
// Greedy verification of a token tree (chzhyang, "Speculative Decoding: ...",
// section 5 DDTree): from the root, follow the child whose token is the
// target's choice at the current node; when no child carries it, that choice
// is the bonus token.  Request b owns nodes off .. off + n_b - 1 (node 0 the
// root), and node i's target row is row off + i.  ReqInfo fields for trees:
// off, k = n_b, a = nodes accepted so far, trow = row of the current node.

// One workgroup: node offsets, every output -1, the row list (all rows) or
// the round-0 list of walking requests (early exit; every request at its root).
__global__ __launch_bounds__(kPlanThreads) void k_tree_plan(Args a) {
  constexpr int kPlanWaves = kPlanThreads / kWave;
  __shared__ long long s_wn[kPlanWaves];
  __shared__ int s_bad, s_na;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid >> 6;
  const bool rounds = a.ee_round >= 0;
  if (tid == 0) {
    s_bad = 0;
    s_na = 0;
  }
  for (long long i = tid; i < a.K; i += kPlanThreads) {
    a.out[i] = -1;
    a.path[i] = -1;
    if (!rounds) a.ws.rowdesc[i] = (uint32_t)i | kGreedyBit;
  }
  for (int i = tid; i < a.B; i += kPlanThreads) a.acc_len[i] = -1;
  __syncthreads();
  long long carry = 0;
  for (int base = 0; base < a.B; base += kPlanThreads) {
    const int b = base + tid;
    long long n = 0;
    if (b < a.B) {
      const int nn = a.num_draft[b];
      if (nn < 1 || nn > a.K) s_bad = 1;
      else n = nn;
    }
    const long long incl = wave_incl_scan_ll(n, lane);
    if (lane == kWave - 1) s_wn[wv] = incl;
    __syncthreads();
    long long pre = 0, tot = 0;
    for (int q = 0; q < kPlanWaves; ++q) {
      if (q < wv) pre += s_wn[q];
      tot += s_wn[q];
    }
    const long long off = carry + pre + incl - n;
    if (b < a.B) {
      ReqInfo r;
      r.off = (int)off;
      r.k = (int)n;
      r.greedy = 1;
      r.a = 0;
      r.kind = KIND_NONE;
      r.y = -1;
      r.trow = (int)off;
      r.drow = -1;
      r.Mp = r.Mq = 0.f;
      r.pad0 = r.pad1 = 0;
      r.Sp = r.Sq = 0.0;
      if (rounds && n >= 1) {           // round 0: at the root, whose row the round reads
        const int ia = atomicAdd(&s_na, 1);
        a.ws.alive[ia] = b;
        a.ws.rows_r[ia] = (uint32_t)off;
      }
      a.ws.req[b] = r;
    }
    carry += tot;
    __syncthreads();
  }
  if (tid == 0) {
    const bool bad = s_bad != 0 || carry != a.K;
    Header* h = a.ws.hdr;
    h->error = bad ? 1 : 0;
    h->n_rows = bad ? 0 : a.K;
    h->n_units = 0;
    h->n_stoch = 0;
    h->n_alive3[0] = (rounds && !bad) ? s_na : 0;   // (list order is free)
    h->n_rows3[0] = (rounds && !bad) ? s_na : 0;
    h->n_alive3[1] = 0;
    h->n_rows3[1] = 0;
  }
}

// 0 <= parent < node for every non-root node of the request (one wavefront).
__device__ bool tree_parents_ok(const Args& a, const ReqInfo& R, int lane) {
  bool bad = false;
  for (int i = 1 + lane; i < R.k; i += kWave) {
    const int p = a.parent[R.off + i];
    bad |= (p < 0 || p >= i);
  }
  return !__any(bad);
}

// Lexicographic (max, lowest id) over the unit partials P[0 .. nseg) of one
// row: lanes over units, then a wavefront reduction (exact in any order).
__device__ int wave_row_argmax(const Partial* P, int nseg, int lane) {
  float bm = -INFINITY;
  int bi = INT_MAX;
  for (int s = lane; s < nseg; s += kWave) {
    const Partial p = P[s];
    if (p.m > bm || (p.m == bm && p.idx < bi)) {
      bm = p.m;
      bi = p.idx;
    }
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    const float ob = __shfl_xor(bm, o);
    const int oi = __shfl_xor(bi, o);
    if (ob > bm || (ob == bm && oi < bi)) {
      bm = ob;
      bi = oi;
    }
  }
  return bi;
}

// One step of the walk for request b at its current node (global row trow),
// whose unit partials are P: the target's choice, then the lowest-index child
// of the node carrying that token.  Lane 0 writes the path and token slots.
// Returns the child's local index, or -1 when the walk ends (acc_len written).
__device__ int tree_step(const Args& a, int b, const ReqInfo& R, const Partial* P, int t,
                         int lane) {
  const int cur = R.trow - R.off;
  const int choice = wave_row_argmax(P, a.nseg, lane);
  int follow = -1;
  if (choice != INT_MAX) {
    for (int i0 = cur + 1; i0 < R.k && follow < 0; i0 += kWave) {
      const int i = i0 + lane;
      const bool m = i < R.k && a.parent[R.off + i] == cur && a.tokens[R.off + i] == choice;
      const unsigned long long hit = __ballot(m);
      if (hit) follow = i0 + __ffsll((long long)hit) - 1;
    }
  }
  if (lane == 0) {
    a.path[R.off + t] = cur;
    a.out[R.off + t] = (choice == INT_MAX) ? -1 : choice;
    if (follow < 0) a.acc_len[b] = t;
  }
  return follow;
}

// All-rows walk: one wavefront per request after k_stats has summarised every
// node row.
__global__ __launch_bounds__(kBlock) void k_tree_walk(Args a) {
  if (a.ws.hdr->error) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int gw = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int W = gridDim.x * kWavesPerBlock;
  for (int b = gw; b < a.B; b += W) {
    ReqInfo R = a.ws.req[b];
    if (!tree_parents_ok(a, R, lane)) continue;   // outputs keep -1
    for (int t = 0;; ++t) {             // every step moves to a higher node index
      const int f = tree_step(a, b, R, a.ws.pt + (int64_t)R.trow * a.nseg, t, lane);
      if (f < 0) break;
      R.trow = R.off + f;
    }
  }
}

// Early-exit rounds.  Round r covers the walk's steps [P_r, P_(r+1)) with
// P = 0, 1, 2, 4, 8, ... (the last window ends at max_depth + 1): k_tree_round
// streams the rows listed for the round (argmax units of kTreeSegBytes, so
// that the few rows of a round still spread over every CU; partials per node
// row), then one wavefront per walking request takes the window's steps and,
// if it is still walking, lists its new current node and the descendants the
// next window can reach.  Lists of rows and of walking requests rotate over
// three buffers; k_tree_round of round r clears the counts k_tree_step_round
// of round r fills.
template <class L>
__global__ __launch_bounds__(kBlock) void k_tree_round(Args a) {
  using Elem = typename L::Elem;
  const int lane = threadIdx.x & (kWave - 1);
  const int gw = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int W = gridDim.x * kWavesPerBlock;
  const int j = a.ee_round;
  const int cur = j % 3, nxt = (j + 1) % 3;
  Header* hdr = a.ws.hdr;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    hdr->n_alive3[nxt] = 0;
    hdr->n_rows3[nxt] = 0;
  }
  const int n_units = hdr->n_rows3[cur] * a.nseg;
  const uint32_t* rows = a.ws.rows_r + (int64_t)cur * a.K;
  const Elem* tgt = static_cast<const Elem*>(a.target);
  for (int u = gw; u < n_units; u += W) {
    const int ri = u / a.nseg;
    const int seg = u - ri * a.nseg;
    const int row = (int)rows[ri];
    const int s0 = seg * a.seg;
    const int s1 = min(s0 + a.seg, a.V);
    argmax_unit<L>(tgt + (int64_t)row * a.tld, s0, s1, lane,
                   a.ws.pt + (int64_t)row * a.nseg + seg);
  }
}

// Node i (local, i > c) lies at most depth levels below node c: its parent
// chain reaches c within depth links (parents have lower indices, so the
// chain can stop as soon as it drops below c).
__device__ __forceinline__ bool tree_below(const Args& a, int off, int c, int i, int depth) {
  int p = i;
  for (int s = 0; s < depth; ++s) {
    p = a.parent[off + p];
    if (p == c) return true;
    if (p < c) return false;
  }
  return false;
}

// List node c of request R and its descendants up to depth levels below it
// (the rows a window of depth + 1 steps from c can visit) for the next round.
__device__ void tree_list_rows(const Args& a, const ReqInfo& R, int c, int depth, int nxt,
                               int lane) {
  int cnt = 1;
  if (depth > 0)
    for (int i0 = c + 1; i0 < R.k; i0 += kWave) {
      const int i = i0 + lane;
      cnt += __popcll(__ballot(i < R.k && tree_below(a, R.off, c, i, depth)));
    }
  int ir = 0;
  if (lane == 0) ir = atomicAdd(&a.ws.hdr->n_rows3[nxt], cnt);
  ir = __shfl(ir, 0);
  uint32_t* rows = a.ws.rows_r + (int64_t)nxt * a.K;
  if (lane == 0) rows[ir] = (uint32_t)(R.off + c);
  int pos = ir + 1;
  if (depth > 0)
    for (int i0 = c + 1; i0 < R.k; i0 += kWave) {
      const int i = i0 + lane;
      const bool d = i < R.k && tree_below(a, R.off, c, i, depth);
      const unsigned long long m = __ballot(d);
      if (d) rows[pos + __popcll(m & ((1ull << lane) - 1ull))] = (uint32_t)(R.off + i);
      pos += __popcll(m);
    }
}

__global__ __launch_bounds__(kBlock) void k_tree_step_round(Args a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int gw = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int W = gridDim.x * kWavesPerBlock;
  const int j = a.ee_round;
  const int cur = j % 3, nxt = (j + 1) % 3;
  Header* hdr = a.ws.hdr;
  const int nal = hdr->n_alive3[cur];
  for (int w = gw; w < nal; w += W) {
    const int b = a.ws.alive[(int64_t)cur * a.B + w];
    ReqInfo R = a.ws.req[b];
    if (a.ee_lo == 0 && !tree_parents_ok(a, R, lane)) continue;   // outputs keep -1
    bool walking = true;
    for (int t = a.ee_lo; t < a.ee_hi && walking; ++t) {
      const int f = tree_step(a, b, R, a.ws.pt + (int64_t)R.trow * a.nseg, t, lane);
      if (f < 0) {
        walking = false;                // acc_len written by tree_step
      } else if (t == a.max_k) {
        // the walk would accept more than max_depth nodes: an input error, the
        // request reports -1 everywhere
        for (int i = lane; i <= t; i += kWave) {
          a.path[R.off + i] = -1;
          a.out[R.off + i] = -1;
        }
        walking = false;
      } else {
        R.trow = R.off + f;
      }
    }
    if (!walking) continue;
    if (lane == 0) {
      a.ws.req[b].trow = R.trow;
      const int ia = atomicAdd(&hdr->n_alive3[nxt], 1);
      a.ws.alive[(int64_t)nxt * a.B + ia] = b;
    }
    tree_list_rows(a, R, R.trow - R.off, a.ee_nhi - a.ee_hi - 1, nxt, lane);
  }
}

// ------------------------------------------------------------------ token trees (host)
struct TreeSizes {
  size_t off_hdr, off_req, off_rowdesc, off_pt, off_alive, off_rows_r, total;
};

bool compute_tree_sizes(long long B, long long N, long long V, TreeSizes* z) {
  if (B < 1 || N < B || V < 1 || V > (1ll << 30)) return false;
  if (N >= (1ll << 29)) return false;
  // 4 KiB units (the rounds) outnumber 32 KiB units (all node rows), so the
  // partials are sized for the former
  const long long ntseg = (V + kTreeSegBytes / 4 - 1) / (kTreeSegBytes / 4);
  if (N * ntseg >= (1ll << 31)) return false;
  const long long npart = N * ntseg;   // every node row, in 32 KiB (all rows) or 4 KiB units
  size_t o = 0;
  z->off_hdr = o; o = align_up(o + sizeof(Header), 256);
  z->off_req = o; o = align_up(o + sizeof(ReqInfo) * (size_t)B, 256);
  z->off_rowdesc = o; o = align_up(o + 4 * (size_t)N, 256);
  z->off_pt = o; o = align_up(o + sizeof(Partial) * (size_t)npart, 256);
  z->off_alive = o; o = align_up(o + 4 * (size_t)(3 * B), 256);
  z->off_rows_r = o; o = align_up(o + 4 * (size_t)(3 * N), 256);
  z->total = o + 256;
  return true;
}

template <class L>
void launch_tree(const Args& a, hipStream_t st, int dev, bool early_exit) {
  static std::atomic<int> occ_stats[64];
  static std::atomic<int> occ_round[64];
  const long long cus = cu_count(dev);
  const int grid_walk = (int)std::max(1ll, std::min(cus * kBlocksPerCU, ((long long)a.B + kWavesPerBlock - 1) / kWavesPerBlock));
  k_tree_plan<<<1, kPlanThreads, 0, st>>>(a);
  if (!early_exit) {
    const long long units = (long long)a.K * a.nseg;
    const long long cap = cus * resident_blocks(occ_stats, k_stats<L>, dev);
    const int grid = (int)std::max(1ll, std::min(cap, (units + kWavesPerBlock - 1) / kWavesPerBlock));
    if (g_ev_begin && g_ev_end) (void)hipEventRecord((hipEvent_t)g_ev_begin, st);
    k_stats<L><<<grid, kBlock, 0, st>>>(a);
    if (g_ev_begin && g_ev_end) (void)hipEventRecord((hipEvent_t)g_ev_end, st);
    k_tree_walk<<<grid_walk, kBlock, 0, st>>>(a);
    return;
  }
  const long long units = (long long)a.K * a.nseg;
  const long long cap = cus * resident_blocks(occ_round, k_tree_round<L>, dev);
  const int grid = (int)std::max(1ll, std::min(cap, (units + kWavesPerBlock - 1) / kWavesPerBlock));
  if (g_ev_begin && g_ev_end) (void)hipEventRecord((hipEvent_t)g_ev_begin, st);
  // windows of steps [P_r, P_(r+1)), P = 0, 1, 2, 4, 8, ..., up to max_depth + 1
  const int end = a.max_k + 1;
  auto start = [](int r) { return r == 0 ? 0 : (1 << (r - 1)); };
  for (int r = 0, lo = 0; lo < end; ++r) {
    const int hi = std::min(start(r + 1), end);
    Args ra = a;
    ra.ee_round = r;
    ra.ee_lo = lo;
    ra.ee_hi = hi;
    ra.ee_nhi = std::min(start(r + 2), end);
    k_tree_round<L><<<grid, kBlock, 0, st>>>(ra);
    k_tree_step_round<<<grid_walk, kBlock, 0, st>>>(ra);
    lo = hi;
  }
  if (g_ev_begin && g_ev_end) (void)hipEventRecord((hipEvent_t)g_ev_end, st);
}

int32_t run_tree(const sv_tree_t* tr, int32_t* acc_len, int32_t* path, int32_t* out, void* ws,
                 size_t ws_bytes, void* stream, bool early_exit, int max_depth) {
  if (!tr) return SV_ERR_INVALID_ARG;
  if (early_exit && (max_depth < 0 || max_depth > kMaxEarlyExitRounds)) return SV_ERR_INVALID_ARG;
  const long long B = tr->B, N = tr->N, V = tr->V;
  TreeSizes z;
  if (!compute_tree_sizes(B, N, V, &z)) return SV_ERR_INVALID_ARG;
  if (tr->dtype != SV_F32 && tr->dtype != SV_BF16) return SV_ERR_UNSUPPORTED;
  const int es = tr->dtype == SV_F32 ? 4 : 2;
  if (!tr->num_nodes || !tr->parent || !tr->tokens || !tr->target) return SV_ERR_INVALID_ARG;
  if (!acc_len || !path || !out) return SV_ERR_INVALID_ARG;
  if (tr->target_ld < V || tr->target_ld > (1ll << 40)) return SV_ERR_INVALID_ARG;
  if ((uintptr_t)tr->target % es != 0) return SV_ERR_INVALID_ARG;
  if (!ws) return SV_ERR_WORKSPACE;
  if (ws_bytes < z.total) return SV_ERR_WORKSPACE;

  const uintptr_t wb = align_up((uintptr_t)ws, 256);
  Args a = {};
  a.B = (int)B;
  a.K = (int)N;
  a.V = (int)V;
  a.seg = (early_exit ? kTreeSegBytes : kSegBytes) / es;
  a.nseg = (int)((V + a.seg - 1) / a.seg);
  a.rseg = kRSegBytes / es;
  a.nrseg = (int)((V + a.rseg - 1) / a.rseg);
  a.force_greedy = 1;
  a.tld = tr->target_ld;
  a.target = tr->target;
  a.num_draft = tr->num_nodes;
  a.tokens = tr->tokens;
  a.parent = tr->parent;
  a.acc_len = acc_len;
  a.out = out;
  a.path = path;
  set_scale(1.0, &a.c, &a.c64);
  a.ws.hdr = reinterpret_cast<Header*>(wb + z.off_hdr);
  a.ws.req = reinterpret_cast<ReqInfo*>(wb + z.off_req);
  a.ws.rowdesc = reinterpret_cast<uint32_t*>(wb + z.off_rowdesc);
  a.ws.pt = reinterpret_cast<Partial*>(wb + z.off_pt);
  a.ws.alive = reinterpret_cast<int*>(wb + z.off_alive);
  a.ws.alive_e = nullptr;
  a.ws.rows_r = reinterpret_cast<uint32_t*>(wb + z.off_rows_r);
  a.rowlist = a.ws.rowdesc;
  a.rowcount = &a.ws.hdr->n_rows;
  a.ee_round = early_exit ? 0 : -1;
  a.ee_lo = a.ee_hi = a.ee_nhi = 0;
  a.max_k = early_exit ? max_depth : 0;

  const bool vec = ((uintptr_t)tr->target % 16 == 0) && ((tr->target_ld * es) % 16 == 0);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SV_ERR_HIP;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (tr->dtype == SV_F32) {
    if (vec) launch_tree<F32>(a, st, dev, early_exit);
    else launch_tree<Scalar<F32>>(a, st, dev, early_exit);
  } else {
    if (vec) launch_tree<BF16>(a, st, dev, early_exit);
    else launch_tree<Scalar<BF16>>(a, st, dev, early_exit);
  }
  if (hipGetLastError() != hipSuccess) return SV_ERR_HIP;
  return SV_OK;
}

}  // namespace

extern "C" size_t spec_verify_tree_workspace_bytes(int32_t B, int32_t N, int32_t V) {
  TreeSizes z;
  return compute_tree_sizes(B, N, V, &z) ? z.total : 0;
}
extern "C" int32_t spec_verify_tree_greedy(const sv_tree_t* tree, int32_t* accepted_len,
                                           int32_t* path_nodes, int32_t* out_tokens,
                                           void* workspace, size_t workspace_bytes, void* stream) {
  return run_tree(tree, accepted_len, path_nodes, out_tokens, workspace, workspace_bytes, stream,
                  false, 0);
}
extern "C" int32_t spec_verify_tree_greedy_early_exit(const sv_tree_t* tree, int32_t max_depth,
                                                      int32_t* accepted_len, int32_t* path_nodes,
                                                      int32_t* out_tokens, void* workspace,
                                                      size_t workspace_bytes, void* stream) {
  return run_tree(tree, accepted_len, path_nodes, out_tokens, workspace, workspace_bytes, stream,
                  true, max_depth);
}
