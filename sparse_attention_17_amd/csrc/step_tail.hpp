// Host interface of the fused decode-step tail (step_tail.hip): the per-row
// top-k pick, the CSA and HCA split attention and the split merges of one
// decode step in a single launch.
#pragma once
#include "launch.hpp"

namespace csa {

// Bytes of control words the tail keeps at the front of the step workspace
// (zero before the first launch; every launch leaves them zero).  One fixed
// size for every batch (the tail handles batches up to 1580 sequences).
size_t decode_tail_ctl_bytes();
// Whether the two attention problems of a step take the fused tail (one
// query token per sequence, bf16, head dim 128, both split, same wave shape).
bool decode_tail_supported(const AttendArgs& csa_a, const AttendArgs& hca_a);
// Enqueues the tail.  picks: the row picks run as tasks of the tail (the
// indexer's score kernel must already be enqueued on `st`); otherwise the
// index rows must already be enqueued (score kernel and row pick).
hipError_t launch_decode_tail(const IndexerArgs& ix, const AttendArgs& csa_a, const AttendArgs& hca_a,
                              void* ctl, unsigned long long* counters, bool picks, hipStream_t st);

}  // namespace csa
