"""The stamped-slot feature hand-off (tap_send / tap_recv) on one GPU:
payloads arrive bit-exact in order of their stamps, a consumer started
before its producer waits for the stamp, and the bounded waits report a
missing or overwritten sequence instead of copying."""

import pytest

torch = pytest.importorskip("torch")

from gpu_util import say  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import branch_aware_causal_amd  # noqa: F401


def mailbox(nslots, slot_bytes):
    slots = torch.zeros(nslots, slot_bytes, dtype=torch.uint8, device="cuda")
    stamps = torch.zeros(nslots, dtype=torch.int64, device="cuda")
    return slots, stamps


def rand_bytes(n, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randint(0, 256, (n,), generator=g, dtype=torch.int32, device="cuda").to(torch.uint8)


@pytest.mark.parametrize("nbytes", [16, 1000003, 8 << 20])
def test_send_then_receive_is_bit_exact(nbytes):
    from branch_aware_causal_amd import tap_recv, tap_send
    say(f"case tap send/recv nbytes={nbytes}")
    slots, stamps = mailbox(2, 8 << 20)
    payload = rand_bytes(nbytes, 1)
    out = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    tap_send(slots, stamps, 1, payload, 7)
    tap_recv(slots, stamps, 1, 7, out, status, spin_limit=1 << 20)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(out, payload)
    assert int(stamps[1].item()) == 7 and int(stamps[0].item()) == 0


def test_consumer_started_first_waits_for_the_stamp():
    """The consumer's stream starts polling before the producer's stream has
    sent anything; it sees the payload only through the stamp."""
    from branch_aware_causal_amd import tap_recv, tap_send
    say("case tap consumer first")
    slots, stamps = mailbox(4, 4 << 20)
    payload = rand_bytes(4 << 20, 2)
    out = torch.zeros_like(payload)
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    prod, cons = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    tap_recv(slots, stamps, 2, 1, out, status, spin_limit=1 << 24, stream=cons)
    # producer work queued behind a few hundred MB of fills so that the
    # consumer is already polling when the payload is written
    with torch.cuda.stream(prod):
        pad = torch.empty(1 << 26, dtype=torch.float32, device="cuda")
        for _ in range(8):
            pad.fill_(1.0)
    tap_send(slots, stamps, 2, payload, 1, stream=prod)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(out, payload)


def test_wait_gives_up_after_its_spin_limit():
    from branch_aware_causal_amd import tap_recv
    say("case tap timeout")
    slots, stamps = mailbox(2, 1 << 16)
    out = torch.full((1 << 16,), 0xAB, dtype=torch.uint8, device="cuda")
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    tap_recv(slots, stamps, 0, 3, out, status, spin_limit=64)    # nothing is ever sent
    torch.cuda.synchronize()
    assert int(status.item()) == 1
    assert bool((out == 0xAB).all())


def test_overwritten_slot_is_reported():
    from branch_aware_causal_amd import tap_recv, tap_send
    say("case tap newer sequence")
    slots, stamps = mailbox(1, 4096)
    out = torch.full((4096,), 0xCD, dtype=torch.uint8, device="cuda")
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    tap_send(slots, stamps, 0, rand_bytes(4096, 3), 5)
    tap_recv(slots, stamps, 0, 4, out, status, spin_limit=64)
    torch.cuda.synchronize()
    assert int(status.item()) == 2
    assert bool((out == 0xCD).all())


def test_ring_of_slots_in_sequence_order():
    """Sequences 1..12 through 4 slots (slot = seq mod 4), each consumed
    before its slot is reused; every payload arrives intact."""
    from branch_aware_causal_amd import tap_recv, tap_send
    say("case tap ring")
    n = 1 << 18
    slots, stamps = mailbox(4, n)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for seq in range(1, 13):
        payload = rand_bytes(n - seq, 10 + seq)
        out = torch.zeros_like(payload)
        tap_send(slots, stamps, seq % 4, payload, seq)
        tap_recv(slots, stamps, seq % 4, seq, out, status, spin_limit=1 << 20)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, seq
        assert torch.equal(out, payload), seq
