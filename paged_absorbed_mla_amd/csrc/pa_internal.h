// Host-side interface between the C-ABI layer and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

// Resolved, validated parameters of one call (host copy).
struct CallGeom {
  int dtype;            // 10 = f16, 16 = bf16
  int H, hs, vhs, bs, bs_log2;
  int do_rotary, interleaved, rd, ro;
  int window;           // < 0 = off
  float softcap;        // <= 0 = off
  float scale;
  int64_t T;
  int B, MB;
  int64_t NB, P;
  int sep;              // 1: separate (grouped-query) layout with a value cache; 0: latent
  int kvh;              // key/value heads (1 in the latent layout); H is a multiple of it
};

// Write phase: one launch per cache (value / value_cache: separate layout only, else null).
hipError_t launch_write(const CallGeom& g, const void* key, const void* value, const void* cos_t,
                        const void* sin_t, const int32_t* slot, const int32_t* cumseq, const int32_t* past,
                        void* cache, void* value_cache, hipStream_t stream);

// Attention kernel configuration chosen for a call.
struct AttnConfig {
  int hsp, vhsp;   // padded head sizes of the compiled instance
  int nw;          // waves per workgroup
  int kt;          // keys per LDS tile
  int wide;        // 0: attn_kernel (32 rows per wave);
                   // 2: attn_mla_kernel (4 waves x 32 rows, query resident in registers)
  int piece_units; // scheduling cost of one extra piece (query load and epilogue), in KV tiles
  int sep;         // separate-layout instance (value rows from the value cache)
  int rows() const { return wide ? 128 : 32 * nw; }
};

// Chooses the instance for a geometry; returns false when no compiled instance fits.
bool choose_config(const CallGeom& g, AttnConfig* cfg);

// Workspace layout derived from the geometry, the config and the grid size.
struct WsLayout {
  int64_t max_mtiles;   // upper bound on query tiles
  int grid;             // workgroups of the attention launch
  int ranges;           // unit ranges of the schedule (one per workgroup)
  int64_t part_cap;     // partial-result slots
  size_t off_header, off_wg_range, off_wg_tile, off_sched, off_mtiles, off_part_ml, off_part_o;
  int64_t sched_ints;   // scheduler scratch (int32) when it does not fit its LDS
  size_t off_qfrag;     // query in the four-wave kernel's fragment order, RoPE applied [T * H][hsp] (0: none)
  int64_t part_slot;    // partial-output elements between slots (bf16 or f32, by output type)
  int part_row;         // partial-output elements between rows
  size_t total;
};

// Workgroups the attention kernel can keep resident per CU (cached per device).
hipError_t attn_occupancy(const CallGeom& g, const AttnConfig& cfg, int device, int* blocks_per_cu);

WsLayout plan_workspace(const CallGeom& g, const AttnConfig& cfg, int num_cus, int blocks_per_cu, bool split_kv);

// Write phase carried by the attention phase's schedule launch (the fused
// call): key rows [T, kvh * hs] into key_cache at slot_mapping (RoPE per key
// head), and in the separate layout value rows into value_cache.
struct FusedWrite {
  const void* key;
  const int32_t* slot_mapping;
  void* key_cache;
  const void* value;    // separate layout: value rows [T, kvh * vhs], stored unrotated (else null)
  void* value_cache;
};

// Attention phase: schedule, attention, combine (three launches). `ev`: null, or
// two events recorded right before and after the attention kernel's launch.
// `fw`: null, or the write phase to run in the schedule launch (before the
// attention kernel reads the cache).
hipError_t launch_attention(const CallGeom& g, const AttnConfig& cfg, const WsLayout& ws, bool split_kv,
                            const void* query, const void* cache, const void* value_cache, const void* cos_t,
                            const void* sin_t, const int32_t* cumseq, const int32_t* past,
                            const int32_t* block_table, void* out, void* workspace, hipStream_t stream,
                            const hipEvent_t* ev, const FusedWrite* fw = nullptr);

}  // namespace pa
