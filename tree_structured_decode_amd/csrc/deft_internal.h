// Internal declarations shared by the host planner and the HIP launchers.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "deft.h"

namespace deft {

// Largest chunk the attention kernels stage (token row indices and masks of
// one chunk live in LDS).
constexpr int kMaxChunkTokens = 4096;
constexpr int kPageSize = 16;

// Row blocking of the work lists.  A "row" is one (slot, query head) pair of
// a chunk: rows of chunk c are r = j * G + hh for the chunk's j-th slot and
// the hh-th query head of the KV head being processed (G = Hq / Hkv).
constexpr int kMfmaRows = 64;      // rows per MFMA work item (4 tiles of 16)
constexpr int kMfmaWideRows = 128; // rows per wide MFMA work item (groups of more than kMfmaRows rows)
constexpr int kMfmaGroupRows = 256; // rows per whole-group MFMA work item (no token split)
constexpr int kMfmaMinRows = 1;    // default rows a bf16 chunk needs to use MFMA (every chunk)
constexpr int kValuRows = 8;       // rows per VALU work item
constexpr int64_t kMaxQueryRows = int64_t{1} << 28;       // num_queries * num_q_heads < this
constexpr int64_t kMaxPartialBlocks = (int64_t{1} << 23) - 1; // grid x 512 threads < 2^32

struct WorkItem {                  // two int4 on the device
  int32_t chunk;
  int32_t row_begin;
  int32_t row_count;
  int32_t chunk_start;             // copies of the chunk's metadata, so a
  int32_t chunk_len;               // work-group reads one record before it
  int32_t group_offset;            // can start on the chunk's token rows
  int32_t full;
  int32_t logical_start;           // logical index of the chunk's first token
                                   // when its tokens are consecutive logical
                                   // tokens (no flat-to-logical lookup), else -1
};
static_assert(sizeof(WorkItem) == 32, "work items are read as two int4");

// Offsets (in 4-byte words) of each array inside the device image.
struct ImageLayout {
  size_t chunk_start, group_offsets, chunk_full, slot_query, slot_mask, flat_to_logical,
      query_slot_offsets, query_slots, mfma_items, valu_items, tickets, status, merge_slots, total_words;
  int32_t n_mfma_group, n_mfma_wide, n_mfma, n_valu;   // mfma_items: group, wide, then 64-row items
  // Merge lists at a fixed stride (each query's slots, padded with -1), so
  // the merge reads a query's slot ids without first reading its offsets;
  // 0 when the plan's slot counts are too uneven for that (CSR lists only).
  int32_t merge_stride;
  int32_t max_valu_rows;   // largest row count of a VALU work item (picks the kernel's row capacity)
};

void set_error(const std::string& msg);
int fail(int code, const std::string& msg);

}  // namespace deft

struct deft_plan {
  int32_t num_nodes = 0, num_queries = 0, chunk_tokens = 0, total_tokens = 0;
  int32_t num_chunks = 0, num_slots = 0, mask_words = 0;
  std::vector<int32_t> node_start, flat_node_order, node_flat_start, flat_to_logical;
  std::vector<int32_t> chunk_start, group_offsets, slot_query, query_slot_offsets, query_slots;
  std::vector<uint32_t> slot_mask;
  std::vector<uint8_t> chunk_full;

  bool query_centric = false;   // built by deft_plan_create_query_centric

  // Device image for the last uploaded desc.
  bool uploaded = false;
  deft_attn_desc desc{};
  void* dev = nullptr;
  size_t dev_bytes = 0;
  deft::ImageLayout layout{};
  std::vector<int32_t> staging;   // host source of the last upload's copy
  void* staging_done = nullptr;   // hipEvent_t recorded after that copy
};

namespace deft {
// Validates desc against the plan; fills the work lists and layout for it.
int build_image(deft_plan* p, const deft_attn_desc* desc, std::vector<int32_t>* image,
                ImageLayout* layout);
int check_desc(const deft_plan* p, const deft_attn_desc* desc);
// Compute units of the current device (256, the MI355X count, when it cannot
// be queried); the planner sizes its work items to it.
int device_cu_count();
// Waits for the last upload's copy out of the staging buffer and releases
// its event (called by deft_plan_destroy).
void release_upload(deft_plan* p);
// Workspace: partial O (bf16 O / l for bf16 inputs, fp32 unnormalised O for
// fp32 inputs), then part_m and part_l, each 256-byte aligned.
// Whether the attention calls' workspace holds bf16 O / l partials (bf16
// inputs without desc->f32_partials) rather than fp32 unnormalised ones.
inline bool bf16_partials(const deft_attn_desc* d) { return d->dtype == DEFT_DTYPE_BF16 && !d->f32_partials; }
size_t partial_o_words(const deft_plan* p, const deft_attn_desc* desc);
size_t workspace_bytes_for(const deft_plan* p, const deft_attn_desc* desc);
}  // namespace deft
