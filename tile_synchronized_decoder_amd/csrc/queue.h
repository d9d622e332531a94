// Host representation of the instruction queue (internal to libmk).
#pragma once
#include <cstdint>
#include <vector>

#include "mk.h"

namespace mk {

enum Op : uint16_t {
  OP_EMBED = 1, OP_QKV = 2, OP_ATTN = 3, OP_COMBINE = 4, OP_OPROJ = 5, OP_GATEUP = 6, OP_DOWN = 7,
  OP_P_EMBED = 8, OP_P_QKV = 9, OP_P_ATTN = 10, OP_P_OPROJ = 11, OP_P_GATEUP = 12, OP_P_DOWN = 13,
  OP_LMHEAD = 14, OP_ARGMAX = 15,
  OP_COUNT = 16
};
constexpr uint32_t kLmTile = 64;            // vocabulary rows per LM-head tile of a loop queue
constexpr uint32_t kPrevStep = 0x80000000u; // wait-range count flag: the previous step's barriers

constexpr uint32_t kMagic = 0x314B4D54u;   // "TMK1"
constexpr uint32_t kVersion = 1;
constexpr int kMaxDecodeRows = 32;
constexpr int kMaxQueues = 1024;

struct Instr {            // 32 bytes, the INSTR record
  uint16_t op, layer;
  uint32_t a0, a1, a2;
  uint32_t wait_off, wait_cnt;
  uint32_t signal;
  uint32_t n_wait;
};
static_assert(sizeof(Instr) == 32, "instruction record is 32 bytes");

struct Range { uint32_t first, count; };
struct Segment { uint32_t op, layer, first, count; };

}  // namespace mk

struct mk_queue {
  mk_config cfg;
  mk_plan plan;
  uint64_t serial = 0;    // unique per queue built in this process (keys the graph cache)
  uint32_t n_splits = 0;
  std::vector<mk::Instr> instr;
  std::vector<mk::Range> waits;
  std::vector<uint32_t> targets;
  std::vector<mk::Segment> segments;
  // byte offsets of the three parts inside the DEVICE image
  size_t dev_instr_off = 0, dev_waits_off = 0, dev_targets_off = 0, dev_bytes = 0;
};

namespace mk {
void set_error(const char* fmt, ...);
void forget_graphs(uint64_t serial);   // drops the HIP graphs captured for a queue
}
