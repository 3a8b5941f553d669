// The fused forward kernel of attn_fwd_kernel.hip compiled a second time,
// for head_dim 64 only, with one 32-row query block per wave (128 query rows
// per workgroup) and 64-key tiles, two operands read ahead.  The offline tile
// sweep (exact_attention_121_amd/tile_sweep.py, every variant held to the
// fp64 oracle first) measured it 14-19 % faster than the two-block form on
// causal problems whose grid of two-block workgroups is small (B=1, H=32,
// N = 1024 and 4096 on MI355X: the heaviest-first causal order needs several
// rounds of workgroups to fill the tail), and slower on large grids and
// without the mask; attn_api.cpp picks between the two at launch
// (forward_d64_one_block in attn_launch.h).
#ifndef ATTN_QB64
#define ATTN_QB64 1
#endif
#ifndef ATTN_BN64
#define ATTN_BN64 64
#endif
#ifndef ATTN_KAHEAD64
#define ATTN_KAHEAD64 2
#endif
#ifndef ATTN_WG64
#define ATTN_WG64 2
#endif
#define ATTN_ONLY_D 64
#define ATTN_FWD_ENTRY launch_forward_d64_one_block

#include "attn_fwd_kernel.hip"
