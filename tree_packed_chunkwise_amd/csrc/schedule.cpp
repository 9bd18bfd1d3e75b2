// schedule.cpp -- launch order of one forward / reverse call of a plan.
//
// The per-round state passes are a sequential chain over each sequence's
// chunks (HARTS Figure 2(c): one packed call per round), so a round with few
// sequences leaves compute units idle; the chunk-parallel passes have no such
// chain.  Each call therefore forks a second stream of the caller's device
// (default priority, created on first use, kept until the process ends) and
// joins it back with events:
//   forward:  chunk pass of round 0's chunks; then round 0 beside the chunk
//             pass of the later rounds' chunks, run round group by round
//             group (a group: consecutive rounds of at least an eighth of
//             all chunks); each round waits only for its own group's pass.
//   reverse:  the gradient-scale words cleared (and the largest leaf-state
//             gradient found); dO of the last round's chunks gathered (the
//             rest on the second stream beside that round); rounds last to
//             first; once
//             the chunks whose rounds are done amount to a quarter of all
//             chunks, their chunk-local gradients run on the second stream
//             beside the remaining rounds; the rest after round 0; the
//             second stream is joined before the fixed-order reductions.
// No kernel reads memory that a kernel running beside it writes, and every
// sum is in a fixed order, so the results do not depend on how the two
// streams interleave (kda_set_overlap(0) makes every call use the caller's
// stream alone, with the same results).  The fork/join sequence of a call is
// enqueued under a per-device lock (its events are reused from call to call).
#include <hip/hip_runtime.h>

#include <atomic>
#include <map>
#include <mutex>
#include <vector>

#include "common.h"
#include "plan.h"

namespace kda {

hipError_t launch_prep(const FwdArgs& a, bool bf16, int BC, int D, int c_begin, int n_chunks,
                       hipStream_t st);
hipError_t launch_fwd_rounds(const FwdArgs& a, bool bf16, int BC, int D, const int* round_ptr_host,
                             int r_begin, int r_end, int max_slices, hipStream_t st);
hipError_t launch_gather_dO(const BwdArgs& a, bool bf16, int BC, int D, int c_begin, int n_chunks,
                            hipStream_t st);
hipError_t launch_bwd_rounds(const BwdArgs& a, bool bf16, int BC, int D, const int* round_ptr_host,
                             int r_begin, int r_end, int max_slices, hipStream_t st);
hipError_t launch_grad(const BwdArgs& a, bool bf16, int BC, int D, int c_begin, int n_chunks,
                       hipStream_t st);
hipError_t launch_reduce(const BwdArgs& a, int D, int n_rep_rows, int n_root, hipStream_t st);
hipError_t launch_scale_words(const BwdArgs& a, size_t n_dhl, hipStream_t st);

namespace {

struct Side {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr;          // caller's stream -> second stream
  hipEvent_t join = nullptr;          // second stream -> caller's stream
  std::vector<hipEvent_t> groups;     // second stream -> caller's stream, per round group
  std::mutex mu;
};

std::mutex g_mu;
std::map<int, Side*> g_side;
std::atomic<int> g_overlap{1};

// Column slices per sequence of a round that runs beside another stream's
// work (measured on the 4-ary tree workload: 2 beats 4 and 8 there, while a
// lone round prefers all D/16).
constexpr int kSlicesBeside = 2;

hipError_t side_of_current_device(Side** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_side.find(dev);
  if (it != g_side.end()) {
    *out = it->second;
    return hipSuccess;
  }
  Side* sd = new Side();
  e = hipStreamCreateWithFlags(&sd->s, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&sd->fork, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&sd->join, hipEventDisableTiming);
  if (e != hipSuccess) {
    if (sd->join) (void)hipEventDestroy(sd->join);
    if (sd->fork) (void)hipEventDestroy(sd->fork);
    if (sd->s) (void)hipStreamDestroy(sd->s);
    delete sd;
    return e;
  }
  g_side[dev] = sd;
  *out = sd;
  return hipSuccess;
}

// `to` waits for everything enqueued on `from` so far
hipError_t order_after(hipEvent_t ev, hipStream_t from, hipStream_t to) {
  hipError_t e = hipEventRecord(ev, from);
  if (e != hipSuccess) return e;
  return hipStreamWaitEvent(to, ev, 0);
}

int round_chunk_begin(const Plan& p, int r) { return p.seq_chunk_ptr[p.round_seq_ptr[r]]; }

hipError_t group_event(Side* sd, size_t i, hipEvent_t* ev) {
  while (sd->groups.size() <= i) {
    hipEvent_t e = nullptr;
    const hipError_t rc = hipEventCreateWithFlags(&e, hipEventDisableTiming);
    if (rc != hipSuccess) return rc;
    sd->groups.push_back(e);
  }
  *ev = sd->groups[i];
  return hipSuccess;
}

#define KDA_TRY(x)                       \
  do {                                   \
    const hipError_t kda_e_ = (x);       \
    if (kda_e_ != hipSuccess) return kda_e_; \
  } while (0)

}  // namespace

void set_overlap(bool on) { g_overlap.store(on ? 1 : 0); }

hipError_t run_fwd(const FwdArgs& a, bool bf16, int BC, int D, const Plan& p, hipStream_t st) {
  const int R = p.n_rounds, nc = p.n_chunks();
  const int* rp = p.round_seq_ptr.data();
  const int c1 = R > 1 ? round_chunk_begin(p, 1) : nc;
  if (c1 == 0 || c1 >= nc || !g_overlap.load()) {  // nothing to overlap, or one stream asked for
    KDA_TRY(launch_prep(a, bf16, BC, D, 0, nc, st));
    return launch_fwd_rounds(a, bf16, BC, D, rp, 0, R, 0, st);
  }
  Side* sd = nullptr;
  KDA_TRY(side_of_current_device(&sd));
  std::lock_guard<std::mutex> lk(sd->mu);
  KDA_TRY(launch_prep(a, bf16, BC, D, 0, c1, st));
  KDA_TRY(order_after(sd->fork, st, sd->s));
  // round groups [gr[i], gr[i + 1]) from round 1 on, each of >= nc / 8 chunks
  std::vector<int> gr{1};
  for (int r = 2; r < R; ++r)
    if (round_chunk_begin(p, r) - round_chunk_begin(p, gr.back()) >= (nc / 8 > 1 ? nc / 8 : 1))
      gr.push_back(r);
  gr.push_back(R);
  const size_t ng = gr.size() - 1;
  for (size_t i = 0; i < ng; ++i) {
    const int cb = round_chunk_begin(p, gr[i]);
    const int ce = gr[i + 1] < R ? round_chunk_begin(p, gr[i + 1]) : nc;
    hipEvent_t ev = nullptr;
    KDA_TRY(group_event(sd, i, &ev));
    KDA_TRY(launch_prep(a, bf16, BC, D, cb, ce - cb, sd->s));
    KDA_TRY(hipEventRecord(ev, sd->s));
  }
  KDA_TRY(launch_fwd_rounds(a, bf16, BC, D, rp, 0, 1, kSlicesBeside, st));
  for (size_t i = 0; i < ng; ++i) {
    KDA_TRY(hipStreamWaitEvent(st, sd->groups[i], 0));
    KDA_TRY(launch_fwd_rounds(a, bf16, BC, D, rp, gr[i], gr[i + 1], kSlicesBeside, st));
  }
  return hipSuccess;
}

hipError_t run_bwd(const BwdArgs& a, bool bf16, int BC, int D, const Plan& p, hipStream_t st) {
  const int R = p.n_rounds, nc = p.n_chunks();
  const int* rp = p.round_seq_ptr.data();
  Side* sd = nullptr;
  if (R > 1 && nc > 0 && g_overlap.load()) KDA_TRY(side_of_current_device(&sd));
  std::unique_lock<std::mutex> lk;
  if (sd) lk = std::unique_lock<std::mutex>(sd->mu);
  // the gradient-scale words (cleared; the largest leaf-state gradient), then
  // the dO tiles, whose gathering also records each round's largest |dO|:
  // the last round's chunks first; with a second stream the rest are
  // gathered there while that round runs
  const size_t n_dhl = a.dh_leaf ? (size_t)p.n_leaf * a.H * D * D : 0;
  KDA_TRY(launch_scale_words(a, n_dhl, st));
  const int cl = R > 0 ? round_chunk_begin(p, R - 1) : nc;
  hipEvent_t gathered = nullptr;
  if (sd && cl > 0) {
    KDA_TRY(launch_gather_dO(a, bf16, BC, D, cl, nc - cl, st));
    KDA_TRY(order_after(sd->fork, st, sd->s));
    KDA_TRY(launch_gather_dO(a, bf16, BC, D, 0, cl, sd->s));
    KDA_TRY(group_event(sd, 0, &gathered));
    KDA_TRY(hipEventRecord(gathered, sd->s));
  } else {
    KDA_TRY(launch_gather_dO(a, bf16, BC, D, 0, nc, st));
  }
  const int group = nc / 4 > 1 ? nc / 4 : 1;
  int ready_end = nc;   // chunks [ready_end, nc) have their gradients launched
  bool forked = false;
  for (int r = R - 1; r >= 0; --r) {
    if (gathered && r == R - 2) KDA_TRY(hipStreamWaitEvent(st, gathered, 0));
    KDA_TRY(launch_bwd_rounds(a, bf16, BC, D, rp, r, r + 1, sd ? kSlicesBeside : 0, st));
    const int cb = round_chunk_begin(p, r);
    if (sd && r > 0 && ready_end - cb >= group) {
      KDA_TRY(order_after(sd->fork, st, sd->s));
      KDA_TRY(launch_grad(a, bf16, BC, D, cb, ready_end - cb, sd->s));
      ready_end = cb;
      forked = true;
    }
  }
  KDA_TRY(launch_grad(a, bf16, BC, D, 0, ready_end, st));
  if (forked) KDA_TRY(order_after(sd->join, sd->s, st));
  return launch_reduce(a, D, (int)p.rep_row.size(), p.n_root, st);
}

}  // namespace kda
