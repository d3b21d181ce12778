// Internal plan representation shared by the host planner and the kernel launchers.
// Not part of the public ABI (include/segpaged.h is).
#pragma once

#include <atomic>
#include <cstdint>
#include <memory>
#include <vector>

#include "segpaged.h"

namespace segpaged {

// SegmentPageTable format, version 1 (documented in segpaged.h).
constexpr int32_t kMagic = 0x53475054;
constexpr int32_t kVersion = 1;
constexpr int kHeaderInts = 16;
constexpr int kSeqInts = 4;
constexpr int kUnitInts = 16;

enum SeqField { S_N = 0, S_Q0 = 1, S_KVOFF = 2, S_QOFF = 3 };
enum UnitField {
  U_KIND = 0, U_B, U_L, U_H, U_N, U_Q0, U_SINK, U_WIN, U_KVLEN, U_NSEG,
  U_S0POS, U_S0LEN, U_S1POS, U_S1LEN, U_PAGEOFF, U_RETROFF
};

// Work lists that follow the table in the device image.
// decode item: unit, slot_lo, slot_hi, gap_lo (0: none), then the unit's b, l, h and
// page_off, so a wave reads one record before its page ids
constexpr int kDecItemInts = 8;
// decode unit: first item, end item, the unit's first output row within its layer
// (b * Hq + h * G), layer
constexpr int kDecUnitInts = 4;
constexpr int kPreItemInts = 2;   // unit, first query position of the tile | kPrecise
// Prefill tiles whose first row sees fewer keys than this take the precise path
// (softmax weights as a sum of two bf16 terms); bit 31 of the item's row marks them.
constexpr int kPreciseKeys = 128;
constexpr int32_t kPrecise = (int32_t)0x80000000u;
constexpr int kPrefillRows = 256; // query rows per prefill tile: G heads x (256 / G) positions
constexpr int kBlockN = 32;       // keys per prefill block
constexpr int kMaxGroup = 16;     // Q heads per KV head the decode kernel supports
constexpr int kSelChunk = 2048;   // keys per workgroup of the top-p masses and first radix pass
constexpr int kCtrInts = 16;      // prefill work counter line per layer (+1 for all layers);
                                  // its first 8 bytes: (launch generation << 32) | next item
constexpr int64_t kDecMaxParts = 16;     // a decode item is dealt to at most 16 waves
// A decode launch of several rounds of waves deals its last items to this many
// waves each; the plan's decode workspace has room for the extra partials of
// one round of 2048 waves (MI355X: 256 compute units x 8 resident waves).
constexpr int32_t kDecTailParts = 4;
constexpr int64_t kDecTailRecords = (2048 / kDecTailParts) * (kDecTailParts - 1);
constexpr int64_t kNoAllocScratchBytes = SEGPAGED_NOALLOC_SCRATCH_BYTES;  // see segpaged.h

struct LayerRange {
  int64_t unit_b, unit_e;   // units
  int64_t page_b, page_e;   // page-id slots of the table
  int64_t retr_b, retr_e;   // retrieval positions
  int64_t dec_b, dec_e;     // decode items
  int64_t pre_b, pre_e;     // prefill items
  int64_t bld_b, bld_e;     // build list: the table page slots that own a distinct page
  int64_t max_unit_items;   // most decode items of one unit
};

}  // namespace segpaged

struct segpaged_plan {
  int32_t B = 0, L = 0, Hq = 0, Hkv = 0, D = 0, P = 0, G = 0, log2P = 0;
  int32_t split = 0;            // decode keys per item
  int64_t num_units = 0, num_pages = 0, pool_pages = 0, num_retr = 0;
  int64_t num_slots = 0;        // page-list entries (num_pages of them own their page)
  int64_t q_rows = 0, kv_rows = 0;
  int64_t off_seqs = 0, off_units = 0, off_pages = 0, off_retr = 0, table_len = 0;
  int64_t off_bld = 0;          // build list (page slots in order), after the table
  int64_t off_decunits = 0, off_dec = 0, off_pre = 0, off_ctr = 0, total_ints = 0;
  int64_t n_dec = 0, n_pre = 0, max_unit_items = 0;
  std::vector<int32_t> buf;                  // device image: table ++ work lists
  std::vector<segpaged::LayerRange> layers;  // per-layer slices of buf
  std::vector<segpaged_stats> stats;         // per-layer work counts
  segpaged_stats total{};
  // append mode (spec.append_capacity > 0): sequences grow after planning
  int64_t append_cap = 0;                    // tokens each sequence may gain
  int64_t append_chunk = 1;                  // most tokens one append adds to a sequence
  std::vector<int64_t> n_max;                // per sequence: length limit
  int64_t dec_cap = 0, pre_cap = 0;          // work-list capacities (items)
  int64_t off_app = 0;                       // append list: row offsets [B+1], first positions [B]
  bool app_upload = false;                   // image changed since the last segpaged_append
  std::vector<uint8_t> pages_dirty;          // per layer: a page list rotated
  // prefill launch generation per work counter line (L + 1 lines), see segpaged_prefill
  std::unique_ptr<std::atomic<uint32_t>[]> pre_gen;
};
