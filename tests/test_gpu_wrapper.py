"""The torch wrapper (tensor_adamw_optimizer_amd.AdamW) used the torch way:
.grad attributes, parameter-group dicts, a learning-rate change, the AMP
recipe with clipping, and a checkpoint through torch.save / torch.load
(weights_only=True) -- against the oracle."""
import io

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import bits, n_bit_mismatch, say
from tensor_adamw_optimizer_amd import AdamW

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("state", ["f32", "q8"])
def test_wrapper_amp_clip_checkpoint(state):
    say("case: wrapper", state)
    gen = torch.Generator().manual_seed(51)
    shapes = [(64, 33), (1000,), (7,), (300, 3)]
    dts = [torch.float32, torch.bfloat16, torch.float32, torch.bfloat16]
    p_cpu = [(torch.randn(s, generator=gen) * 0.02).to(d) for s, d in zip(shapes, dts)]
    params = [p.to(DEV) for p in p_cpu]
    groups = [{"params": [params[0], params[2]], "lr": 1e-3, "weight_decay": 0.1},
              {"params": [params[1], params[3]], "lr": 5e-4, "betas": (0.8, 0.99)}]
    opt = AdamW(groups, lr=1e-3, state=state)
    order = [0, 2, 1, 3]                          # the wrapper's tensor order (group by group)
    gdef = [W.Group(lr=1e-3, weight_decay=0.1), W.Group(lr=5e-4, beta1=0.8, beta2=0.99)]
    ref = oracle.OracleAdamW([p_cpu[i].numel() for i in order],
                             ["f32" if dts[i] == torch.float32 else "bf16" for i in order],
                             ["f32" if dts[i] == torch.float32 else "bf16" for i in order],
                             [0, 0, 1, 1], state)
    th_ref = [bits(p_cpu[i]) for i in order]
    fi = torch.zeros(1, device=DEV)
    scale = 1024.0
    inv = torch.tensor([1.0 / scale], device=DEV)
    max_norm = 0.02
    blob = None
    for k in range(1, 9):
        if k == 5:
            # checkpoint, then continue in a fresh optimizer over the same params
            buf = io.BytesIO()
            torch.save(opt.state_dict(), buf)
            buf.seek(0)
            sd = torch.load(buf, weights_only=True)
            opt.close()
            opt = AdamW(groups, lr=1e-3, state=state)
            opt.load_state_dict(sd)
        if k == 6:
            opt.param_groups[0]["lr"] = 2e-3
            gdef[0] = W.Group(lr=2e-3, weight_decay=0.1)
        g_cpu = [(torch.randn(s, generator=gen) * 1e-3 * scale).to(d) for s, d in zip(shapes, dts)]
        for p, g in zip(params, g_cpu):
            p.grad = g.to(DEV)
        if k == 3:
            params[2].grad = None
        fi.zero_()
        norm, coef = opt.clip_grad_norm(max_norm, inv_scale=inv, found_inf=fi)
        opt.step(found_inf=fi, inv_scale=inv, clip_coef=coef)
        g_np = [None if (k == 3 and i == 2) else bits(g_cpu[i]) for i in order]
        found = ref.unscale_check(g_np, 1.0 / scale)
        c = ref.clip_coef(ref.grad_norm(g_np, 1.0 / scale), max_norm)
        torch.cuda.synchronize()
        assert coef.item() == c
        ref.step(th_ref, g_np, gdef, found_inf=found, inv_scale=1.0 / scale, clip_coef=c)
        opt.zero_grad()
    torch.cuda.synchronize()
    assert np.array_equal(bits(opt.steps()), ref.t)
    for j, i in enumerate(order):
        assert n_bit_mismatch(bits(params[i]), th_ref[j]) == 0, i
        m, v = opt.moments(j)
        assert n_bit_mismatch(bits(m), ref.m[j]) == 0 and n_bit_mismatch(bits(v), ref.v[j]) == 0
    opt.close()


def test_wrapper_rejects_sparse_grads_and_reads_steps():
    """A sparse grad cannot go through the dense ABI: the wrapper raises
    ApexwError(APEXW_ESPARSE) before queueing anything; read_steps and the
    "fp32" state alias work."""
    from tensor_adamw_optimizer_amd import _lib as L
    say("case: wrapper sparse grad / read_steps")
    p = torch.zeros(8, 4, device="cuda")
    q = torch.zeros(16, device="cuda")
    opt = AdamW([p, q], lr=1e-3, state="fp32")
    p.grad = torch.ones(8, 4, device="cuda")
    q.grad = torch.ones(16, device="cuda")
    opt.step()
    assert opt.read_steps() == [1, 1]
    p.grad = torch.ones(8, 4, device="cuda").to_sparse()
    with pytest.raises(L.ApexwError) as e:
        opt.step()
    assert e.value.code == L.APEXW_ESPARSE
    assert opt.read_steps() == [1, 1]
    opt.close()


def _inv_scale_apex(scale: float) -> float:
    """inv_scale as the Apex guide, section 4.3, forms it: fp64 reciprocal of
    the scale, rounded once to fp32."""
    return float(np.float32(1.0 / np.float64(np.float32(scale))))


def test_inv_scale_is_the_fp64_reciprocal_rounded_once():
    say("case: apexw_inv_scale")
    from tensor_adamw_optimizer_amd import _lib as L
    rng = np.random.default_rng(62)
    scales = np.concatenate([
        np.float32(2.0) ** np.arange(-20, 25, dtype=np.float32),
        np.float32(np.exp(rng.uniform(-80, 80, 400))),
        np.array([3000.0, 65535.0, 1e-30, 3.0e38, 1.5e-45, 0.0, np.inf, np.nan], np.float32)])
    s_dev = torch.from_numpy(scales.astype(np.float32)).to(DEV)
    out = torch.full_like(s_dev, 7.0)
    st = torch.cuda.current_stream().cuda_stream
    for i in range(scales.size):
        L.apexw_inv_scale(s_dev[i:].data_ptr(), out[i:].data_ptr(), st)
    got = out.cpu().numpy()
    with np.errstate(divide="ignore", over="ignore"):
        want = np.float32(1.0 / scales.astype(np.float64))
    assert np.array_equal(got.view(np.uint32)[~np.isnan(want)], want.view(np.uint32)[~np.isnan(want)])
    assert np.isnan(got[np.isnan(want)]).all()
    # in place (scale and result in one float)
    x = torch.tensor([3000.0], device=DEV)
    L.apexw_inv_scale(x.data_ptr(), x.data_ptr(), st)
    assert x.item() == _inv_scale_apex(3000.0)


@pytest.mark.parametrize("init_scale", [2.0 ** 12, 3000.0])
def test_wrapper_with_lr_scheduler_and_grad_scaler_against_oracle(init_scale):
    """The wrapper as a torch.optim.Optimizer: a StepLR schedule changes lr
    between steps, and torch.amp.GradScaler drives the steps -- the scaler
    hands over its scale and overflow flag, the update unscales in the
    kernel by the library-formed fp64 reciprocal of the scale, and a step
    whose grads hold an inf is skipped on the device (the scaler then halves
    its scale).  A power-of-two scale and one that is not; every step
    against the oracle."""
    say("case: wrapper + StepLR + GradScaler", init_scale)
    gen = torch.Generator().manual_seed(61)
    shapes = [(128, 9), (513,)]
    p_cpu = [(torch.randn(s, generator=gen) * 0.02) for s in shapes]
    params = [p.to(DEV) for p in p_cpu]
    opt = AdamW(params, lr=1e-2, weight_decay=0.05)
    assert isinstance(opt, torch.optim.Optimizer)
    sched = torch.optim.lr_scheduler.StepLR(opt, step_size=2, gamma=0.5)
    scaler = torch.amp.GradScaler("cuda", init_scale=init_scale, growth_interval=1000)
    ref = oracle.OracleAdamW([p.numel() for p in p_cpu], ["f32"] * 2, ["f32"] * 2, [0, 0], "f32")
    th_ref = [bits(p) for p in p_cpu]
    lr = 1e-2
    loss = torch.ones((), device=DEV)
    for k in range(1, 8):
        scaler.scale(loss)                           # as a training loop scales its loss
        scale = scaler.get_scale()
        g_cpu = [torch.randn(s, generator=gen) * 1e-3 for s in shapes]
        for p, g in zip(params, g_cpu):
            p.grad = (g * scale).to(DEV)             # as a scaled backward would leave them
        overflow = k == 4
        if overflow:
            params[1].grad[7] = float("inf")
        scaler.step(opt)
        scaler.update()
        grp = [W.Group(lr=lr, weight_decay=0.05)]
        g_np = [bits(g * scale) for g in g_cpu]
        if overflow:
            g_np[1][7] = np.float32(np.inf)
        ref.step(th_ref, g_np, grp, found_inf=overflow, inv_scale=_inv_scale_apex(scale))
        torch.cuda.synchronize()
        assert opt._inv_buf.item() == _inv_scale_apex(scale)
        for i in range(2):
            assert n_bit_mismatch(bits(params[i]), th_ref[i]) == 0, (k, i)
        if overflow:
            assert scaler.get_scale() == scale / 2
        sched.step()
        lr = opt.param_groups[0]["lr"]
        opt.zero_grad()
    assert list(bits(opt.steps())) == [6, 6]
    assert lr == 1e-2 * 0.5 ** 3
    opt.close()


def test_wrapper_grad_table_checks_and_reuse():
    """A non-contiguous grad is refused before anything is queued;
    step_pointers(None) reuses the previous grad table (persistent grad
    buffers), giving the same result as a step that reads .grad."""
    say("case: wrapper grad table")
    gen = torch.Generator().manual_seed(71)
    p_cpu = [torch.randn(32, 16, generator=gen) * 0.02, torch.randn(300, generator=gen) * 0.02]
    a = [p.to(DEV) for p in p_cpu]
    b = [p.to(DEV) for p in p_cpu]
    opt_a = AdamW(a, lr=1e-2, weight_decay=0.1)
    opt_b = AdamW(b, lr=1e-2, weight_decay=0.1)
    g = [torch.randn(32, 16, generator=gen).to(DEV) * 1e-3, torch.randn(300, generator=gen).to(DEV) * 1e-3]
    a[0].grad = g[0].t().contiguous().t()          # same values, transposed strides
    a[1].grad = g[1].clone()
    with pytest.raises(ValueError):
        opt_a.step()
    assert opt_a.read_steps() == [0, 0]
    for k in range(3):
        for p, x in zip(a, g):
            p.grad = x.clone()
        opt_a.step()
        if k == 0:
            for p, x in zip(b, g):
                p.grad = x                          # persistent buffers, read once
            opt_b.step()
        else:
            opt_b.step_pointers(None)               # the same buffers as the last call
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert n_bit_mismatch(bits(x), bits(y)) == 0
    assert opt_a.read_steps() == opt_b.read_steps() == [3, 3]
    opt_a.close()
    opt_b.close()


def test_flat_grads_match_the_default_path_and_backward_fills_them():
    """flat_grads: every .grad is a view of one buffer per dtype, filled in
    place by backward, zeroed in place by zero_grad; the steps equal those of
    an optimizer that reads .grad every step, and a parameter whose storage
    moved ('p.data = ...') is followed.  Checked against the oracle too."""
    say("case: wrapper flat grads")
    gen = torch.Generator().manual_seed(72)
    shapes = [(37, 11), (1000,), (5,), (64, 64)]
    p_cpu = [torch.randn(s, generator=gen) * 0.02 for s in shapes]
    a = [torch.nn.Parameter(p.to(DEV)) for p in p_cpu]
    b = [torch.nn.Parameter(p.to(DEV)) for p in p_cpu]
    opt_a = AdamW(a, lr=1e-2, weight_decay=0.1)
    opt_b = AdamW(b, lr=1e-2, weight_decay=0.1, flat_grads=True)
    views = [p.grad for p in b]
    assert opt_b.flat_grads_intact()
    assert all(v is not None and v.is_contiguous() and v.data_ptr() % 64 == 0 for v in views)
    ref = oracle.OracleAdamW([p.numel() for p in p_cpu], ["f32"] * 4, ["f32"] * 4, [0] * 4, "f32")
    th_ref = [bits(p) for p in p_cpu]
    xs = [torch.randn(8, 37, generator=gen) for _ in range(5)]
    for k in range(5):
        x = xs[k].to(DEV)

        def loss_of(ps):
            h = (x @ ps[0]).sum(1)                       # [8]
            return (h * ps[1][:8]).sum() + ps[2].square().sum() + (ps[3] * 1e-3).sum()

        opt_a.zero_grad()
        opt_b.zero_grad()
        assert all(p.grad is v for p, v in zip(b, views))
        loss_of(a).backward()
        loss_of(b).backward()
        assert opt_b.flat_grads_intact()
        for p, q in zip(a, b):
            assert n_bit_mismatch(bits(p.grad), bits(q.grad)) == 0
        if k == 3:                                       # storage moves under the optimizer
            for p in (a[1], b[1]):
                p.data = p.data.clone()
            th_dev = [bits(p.detach()) for p in a]
            assert all(n_bit_mismatch(t, r) == 0 for t, r in zip(th_dev, th_ref))
        g_np = [bits(p.grad) for p in a]
        opt_a.step()
        opt_b.step()
        ref.step(th_ref, g_np, [W.Group(lr=1e-2, weight_decay=0.1)])
        torch.cuda.synchronize()
        for i in range(4):
            assert n_bit_mismatch(bits(a[i].detach()), th_ref[i]) == 0, (k, i)
            assert n_bit_mismatch(bits(b[i].detach()), th_ref[i]) == 0, (k, i)
    assert opt_a.read_steps() == opt_b.read_steps() == [5] * 4
    b[2].grad = None
    assert not opt_b.flat_grads_intact()
    with pytest.raises(ValueError):                       # a parameter that changed size
        b[0].data = torch.zeros(3, device=DEV)
        opt_b.step()
    opt_a.close()
    opt_b.close()


def test_flat_grads_broken_contract_is_an_error():
    """With flat_grads, a .grad removed or replaced behind the optimizer's
    back is an error at step(), not a step on buffers no longer written:
    every .grad set to None (what Module.zero_grad does by default) is found
    at the next step, one replaced .grad within a pass over the list; nothing
    is queued by the refused steps."""
    say("case: wrapper flat grads, broken contract")
    ps = [torch.nn.Parameter(torch.randn(n, device=DEV) * 0.02) for n in (300, 7, 4096, 55, 1)]
    opt = AdamW(ps, lr=1e-3, weight_decay=0.1, flat_grads=True)
    before = [p.detach().clone() for p in ps]
    saved = [p.grad for p in ps]
    for p in ps:                                          # Module.zero_grad(set_to_none=True)
        p.grad = None
    with pytest.raises(RuntimeError, match="flat_grads"):
        opt.step()
    for p, g in zip(ps, saved):
        p.grad = g
    opt.step()                                            # intact again: steps
    ps[3].grad = torch.zeros_like(ps[3])                  # one .grad replaced
    with pytest.raises(RuntimeError, match="parameter 3"):
        for _ in range(len(ps)):
            opt.step()
    torch.cuda.synchronize()
    assert opt.read_steps()[3] < len(ps) + 1
    assert all(not torch.equal(p, q) for p, q in zip(ps, before))
    opt.close()


def test_step_hooks_and_profiler_record_like_torch_optimizers():
    """The wrapper runs torch's optimizer step hooks itself: this optimizer's
    and the global pre- and post-hooks are called with (optimizer, args,
    kwargs), a pre-hook may replace the arguments (here it supplies a set
    found_inf flag, so the step is skipped), removed hooks stop being called,
    the profiler records the step under torch's name, and the steps with
    and without hooks are the same updates (against the oracle)."""
    import torch.optim.optimizer as topt
    say("case: wrapper step hooks")
    gen = torch.Generator().manual_seed(5)
    p_cpu = [torch.randn(n, generator=gen) * 0.02 for n in (300, 17)]
    ps = [torch.nn.Parameter(p.to(DEV)) for p in p_cpu]
    opt = AdamW(ps, lr=1e-3, weight_decay=0.1)
    assert getattr(AdamW.step, "hooked", False)          # torch's wrapper is not added
    ref = oracle.OracleAdamW([p.numel() for p in p_cpu], ["f32"] * 2, ["f32"] * 2, [0, 0], "f32")
    th_ref = [bits(p) for p in p_cpu]
    calls = []
    skip = torch.ones(1, dtype=torch.float32, device=DEV)

    def pre(o, args, kwargs):
        calls.append(("pre", o is opt, len(args)))
        if kwargs.get("found_inf") is None and len(calls) == 5:
            kwargs = dict(kwargs, found_inf=skip)        # the second hooked step is skipped
            return args, kwargs
        return None

    def post(o, args, kwargs):
        calls.append(("post", o is opt))

    def gpre(o, args, kwargs):
        calls.append(("gpre", o is opt))

    g_all = []
    for k in range(5):
        g = [torch.randn(p.shape, generator=gen) * 1e-3 for p in p_cpu]
        for p, gg in zip(ps, g):
            p.grad = gg.to(DEV)
        g_all.append([bits(gg) for gg in g])
    h1 = opt.register_step_pre_hook(pre)
    h2 = opt.register_step_post_hook(post)
    h3 = topt.register_optimizer_step_pre_hook(gpre)
    groups = [W.Group(lr=1e-3, weight_decay=0.1)]
    try:
        for k in range(3):
            for p, gg in zip(ps, g_all[k]):
                p.grad = torch.from_numpy(gg).to(DEV)
            opt.step()
            ref.step(th_ref, g_all[k], groups, found_inf=(k == 1))
        assert [c[0] for c in calls] == ["gpre", "pre", "post"] * 3
        assert all(c[1] for c in calls)
    finally:
        h1.remove()
        h2.remove()
        h3.remove()
    n_calls = len(calls)
    with torch.profiler.profile(activities=[torch.profiler.ProfilerActivity.CPU], acc_events=True) as prof:
        for p, gg in zip(ps, g_all[3]):
            p.grad = torch.from_numpy(gg).to(DEV)
        opt.step()
        ref.step(th_ref, g_all[3], groups)
    assert any(e.name == "Optimizer.step#AdamW.step" for e in prof.events())
    for p, gg in zip(ps, g_all[4]):
        p.grad = torch.from_numpy(gg).to(DEV)
    opt.step()                                           # no hooks, no profiler: the fast path
    ref.step(th_ref, g_all[4], groups)
    assert len(calls) == n_calls
    torch.cuda.synchronize()
    for i in range(2):
        assert n_bit_mismatch(bits(ps[i].detach()), th_ref[i]) == 0, i
    assert opt.read_steps() == [4, 4]
    opt.close()


def test_scaler_attributes_on_a_step_without_grads():
    """GradScaler.step hands the optimizer the plain number 0 as found_inf
    when no parameter has a grad; such a step does nothing and is no error."""
    say("case: wrapper, scaler attributes without grads")
    ps = [torch.nn.Parameter(torch.randn(300, device=DEV)), torch.nn.Parameter(torch.randn(7, device=DEV))]
    before = [p.detach().clone() for p in ps]
    opt = AdamW(ps, lr=1e-2, weight_decay=0.1)
    opt.grad_scale = torch.full((1,), 1024.0, device=DEV)
    opt.found_inf = 0
    opt.step()
    torch.cuda.synchronize()
    assert opt.read_steps() == [0, 0]
    assert all(torch.equal(p, q) for p, q in zip(ps, before))
    opt.close()
