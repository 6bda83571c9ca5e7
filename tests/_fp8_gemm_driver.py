"""Drive the fp8 x MXFP4 grouped GEMMs at the c5 shape (T=8192 H=7168 H'=2048 E=384 K=8) on
directly drawn inputs, for hardware-counter runs: route + permute once, then ITERS rounds of
gate/up (rows gathered from x, permuted block-major scales) and down. The inputs are random
e4m3 codes, random e2m1 bytes and constant scales, not the seeded workload (rocprofv3 --pmc
aborts in the workload generator at this size). Not a test; nothing here is checked."""
import sys, os
sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import torch
import mixture_experts_layer_counting_amd as moe
T, H, Hp, E, K = 8192, 7168, 2048, 384, 8
M = T * K
dev = "cuda"
g = torch.Generator(device="cuda").manual_seed(1)
u8 = dict(dtype=torch.uint8, device=dev)
i32 = dict(dtype=torch.int32, device=dev)
f32 = dict(dtype=torch.float32, device=dev)
# fp8 codes in [0, 0x77] with a random sign: finite e4m3fn values
x = (torch.randint(0, 0x78, (T, H), generator=g, **i32) | (torch.randint(0, 2, (T, H), generator=g, **i32) << 7)).to(torch.uint8)
x_sf = torch.full((T, H // 128), 2.0 ** -6, **f32)
logits = torch.randn((T, E), generator=g, **f32)
wg = torch.randint(0, 256, (E, Hp, H // 2), generator=g, **i32).to(torch.uint8)
wu = torch.randint(0, 256, (E, Hp, H // 2), generator=g, **i32).to(torch.uint8)
wd = torch.randint(0, 256, (E, H, Hp // 2), generator=g, **i32).to(torch.uint8)
sg = torch.full((E, H // 32, Hp), 124, **u8)
su = torch.full((E, H // 32, Hp), 124, **u8)
sd = torch.full((E, Hp // 32, H), 124, **u8)
topk_idx = torch.empty((T, K), **i32); topk_w = torch.empty((T, K), **f32)
counts = torch.empty(E, **i32); cu = torch.empty(E + 1, **i32); pos = torch.empty((T, K), **i32)
row_src = torch.empty(M, **i32)
x_perm_sf = torch.empty((H // 128, M), **f32)
nws = moe.moe_permute_workspace_bytes(T, E, K)
ws = torch.empty(nws, **u8)
h = torch.empty((M, Hp), **u8); h_sf = torch.empty((Hp // 128, M), **f32)
y = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
torch.cuda.synchronize()
print("[drv] inputs ready", flush=True)
moe.moe_route_permute(logits, x, x_sf, moe.MOE_FP8_E4M3, T, H, E, K, 1, topk_idx, topk_w, counts, cu, pos,
                      row_src, None, None, x_perm_sf, ws, nws)
for it in range(int(os.environ.get("ITERS", "4"))):
    moe.moe_ffn_gate_up_gather(x, None, x_perm_sf, moe.MOE_FP8_E4M3, row_src, T, K, cu, M, E, H, Hp, wg, wu,
                               sg, su, moe.MOE_MXFP4, h, h_sf)
    moe.moe_ffn_down(h, h_sf, moe.MOE_FP8_E4M3, cu, M, E, H, Hp, wd, sd, moe.MOE_MXFP4, y, moe.MOE_BF16)
torch.cuda.synchronize()
print("[drv] done", int(counts.sum()), float(y[:64].float().abs().sum()), flush=True)
