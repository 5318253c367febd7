// Page-record layout of the paged int8 KV cache (host and device).
//
// A page holds 16 consecutive tokens of one KV slot of one sequence (the
// fixed-size blocks of PagedAttention: "Como funciona a inferência de IA",
// section on what production inference servers do, item 1).  One record keeps
// the int8 K codes, the int8 V codes and the per-token fp32 scales of K and V
// together, so a page read brings everything the attention of those 16 keys
// needs.
//
//   [ K codes : 16*D bytes | V codes : 16*D bytes | sK : 16 f32 | sV : 16 f32 ]
//
// The byte order inside the K and V blocks is chosen for the gfx950 16x16x32
// matrix-core instructions: lane l (i = l % 16, g = l / 16) of a wavefront
// reads 16 contiguous bytes at offset 16*l (+1024 for the second half at
// D = 128), and those bytes are exactly that lane's operand:
//   K block: lane (i, g) gets token i, channels g*D/4 + 16h .. g*D/4 + 16h + 15
//            in 1 KiB piece h (the QK^T operand: keys are the M index,
//            channels the K index; 8 bytes make one 16x16x32 step);
//   V block: lane (i, g) gets, for 4 channel tiles t, channel 16t + i of the
//            tokens 4g .. 4g+3 (the PV operand: channels are the M index,
//            keys the K index).
// The result is that every operand load is perfectly coalesced (a wavefront
// reads 1 KiB of consecutive bytes per instruction) and needs no LDS
// transpose.
//
// K and V codes are both stored with the sign bit flipped (byte = code xor
// 0x80 = code + 128, an unsigned byte): the fp16 operand conversion places
// that byte under a fixed exponent as it is, with no per-dword fix-up in the
// attention loop.
#pragma once
#include <stdint.h>

#ifdef __HIPCC__
#define MQA_HD __host__ __device__
#else
#define MQA_HD
#endif

namespace mqa {

constexpr int kPageTokens = 16;

MQA_HD constexpr int page_bytes(int D) { return 32 * D + 128; }

// Offset of K code (token j, channel c) inside a record.
MQA_HD constexpr int k_code_offset(int D, int j, int c) {
  // channels per lane group CH = D/4; within the group w = c % CH: half
  // w / 16 selects the 1 KiB half, w % 16 the byte inside the lane's 16 bytes.
  return ((c % (D / 4)) >> 4) * 1024 + (c / (D / 4)) * 256 + j * 16 + ((c % (D / 4)) & 15);
}

// Offset of V code (token j, channel c) inside a record.
MQA_HD constexpr int v_code_offset(int D, int j, int c) {
  // channel tile t = c / 16, lane i = c % 16, lane group g = j / 4, r = j % 4
  return 16 * D + ((c >> 4) >> 2) * 1024 + (j >> 2) * 256 + (c & 15) * 16 +
         ((c >> 4) & 3) * 4 + (j & 3);
}

// Stored byte of a K or V code c (-127..127): c + 128.
MQA_HD constexpr uint8_t code_byte(int c) { return (uint8_t)(c ^ 0x80); }

MQA_HD constexpr int k_scale_offset(int D, int j) { return 32 * D + 4 * j; }
MQA_HD constexpr int v_scale_offset(int D, int j) { return 32 * D + 64 + 4 * j; }

}  // namespace mqa
